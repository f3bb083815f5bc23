// C ABI of libspattn: argument validation, workspace sizing and dispatch.
// Validation runs entirely on the host before any HIP call, so every
// argument error is reported without touching a device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/spattn.h"
#include "internal.h"
#include "api_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int elem_size(int dt) {
  switch (dt) {
    case SPATTN_F32: return 4;
    case SPATTN_BF16: return 2;
    case SPATTN_FP8_E4M3: return 1;
    case SPATTN_I32: return 4;
  }
  return 0;
}

// basic structural checks; `aligned16` requires 16-byte aligned rows
int check_tensor(const spattn_tensor* t, const char* name, int ndim, bool aligned16) {
  if (!t) return fail(SPATTN_ERR_INVALID_ARG, "%s: null tensor", name);
  if (!t->data) return fail(SPATTN_ERR_INVALID_ARG, "%s: null data pointer", name);
  if (t->ndim != ndim) return fail(SPATTN_ERR_INVALID_ARG, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  if (!elem_size(t->dtype)) return fail(SPATTN_ERR_INVALID_ARG, "%s: unknown dtype %d", name, t->dtype);
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(SPATTN_ERR_INVALID_ARG, "%s: negative extent", name);
    if (t->stride[i] < 0) return fail(SPATTN_ERR_INVALID_ARG, "%s: negative stride", name);
    if (t->shape[i] > (int64_t)1 << 31) return fail(SPATTN_ERR_UNSUPPORTED, "%s: extent too large", name);
  }
  if (t->shape[ndim - 1] > 1 && t->stride[ndim - 1] != 1)
    return fail(SPATTN_ERR_INVALID_ARG, "%s: innermost dimension must be contiguous", name);
  if (aligned16) {
    const int es = elem_size(t->dtype);
    if (((uintptr_t)t->data) % 16) return fail(SPATTN_ERR_INVALID_ARG, "%s: data not 16-byte aligned", name);
    for (int i = 0; i < ndim - 1; ++i)
      if ((t->stride[i] * es) % 16) return fail(SPATTN_ERR_INVALID_ARG, "%s: stride %d not a multiple of 16 bytes", name, i);
  }
  return SPATTN_OK;
}

sp::View4 view(const spattn_tensor* t) {
  sp::View4 v{};
  v.p = t->data;
  v.dt = t->dtype;
  for (int i = 0; i < 4; ++i) {
    v.n[i] = i < t->ndim ? t->shape[i] : 1;
    v.s[i] = i < t->ndim ? t->stride[i] : 0;
  }
  return v;
}

std::mutex g_dev_mu;
int g_dev_state[64];   // 0 unknown, 1 ok, 2 unsupported

int device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(SPATTN_ERR_NO_DEVICE, "no HIP device available");
  }
  if (dev >= 64) return fail(SPATTN_ERR_NO_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(SPATTN_ERR_NO_DEVICE, "cannot query device %d", dev);
    }
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  if (g_dev_state[dev] != 1) return fail(SPATTN_ERR_NO_DEVICE, "device %d is not gfx950", dev);
  return SPATTN_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(SPATTN_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return SPATTN_OK;
}

// ------------------------------------------------------------------ indexer
int check_indexer(const spattn_indexer* ix, int64_t* B, int64_t* Nq, int64_t* ctx, int64_t* G_sel) {
  if (!ix) return fail(SPATTN_ERR_INVALID_ARG, "indexer: null");
  int rc;
  if ((rc = check_tensor(&ix->q_idx, "q_idx", 4, true))) return rc;
  if ((rc = check_tensor(&ix->k_idx, "k_idx", 4, true))) return rc;
  const spattn_tensor& q = ix->q_idx;
  const spattn_tensor& k = ix->k_idx;
  if (q.dtype != SPATTN_F32 && q.dtype != SPATTN_BF16)
    return fail(SPATTN_ERR_UNSUPPORTED, "q_idx dtype must be f32 or bf16");
  if (k.dtype != SPATTN_F32 && k.dtype != SPATTN_BF16 && k.dtype != SPATTN_FP8_E4M3)
    return fail(SPATTN_ERR_UNSUPPORTED, "k_idx dtype must be f32, bf16 or fp8");
  if (q.dtype == SPATTN_F32 && k.dtype != SPATTN_F32)
    return fail(SPATTN_ERR_UNSUPPORTED, "f32 q_idx requires f32 k_idx");
  if (q.shape[0] != k.shape[0]) return fail(SPATTN_ERR_INVALID_ARG, "q_idx/k_idx batch mismatch");
  if (q.shape[3] != k.shape[3]) return fail(SPATTN_ERR_INVALID_ARG, "q_idx/k_idx head dim mismatch");
  const int64_t H_I = q.shape[2], d_I = q.shape[3];
  if (d_I < 1 || d_I > 256) return fail(SPATTN_ERR_UNSUPPORTED, "d_I must be in 1..256");
  if (ix->score_mode != SPATTN_SCORE_DOT && ix->score_mode != SPATTN_SCORE_WEIGHTED_RELU)
    return fail(SPATTN_ERR_INVALID_ARG, "unknown score mode %d", ix->score_mode);
  const int hpg = ix->heads_per_group;
  if (hpg < 1 || H_I % hpg) return fail(SPATTN_ERR_INVALID_ARG, "heads_per_group must divide H_I");
  if (ix->score_mode == SPATTN_SCORE_DOT && hpg != 1)
    return fail(SPATTN_ERR_INVALID_ARG, "DOT mode needs heads_per_group = 1");
  if ((int64_t)hpg * d_I > 4096) return fail(SPATTN_ERR_UNSUPPORTED, "heads_per_group * d_I > 4096");
  if (hpg > 64) return fail(SPATTN_ERR_UNSUPPORTED, "heads_per_group > 64");
  const int64_t G = H_I / hpg;
  if (k.shape[2] != 1 && k.shape[2] != G)
    return fail(SPATTN_ERR_INVALID_ARG, "k_idx heads must be 1 or the number of selection groups");
  if (ix->score_mode == SPATTN_SCORE_WEIGHTED_RELU) {
    const spattn_tensor& w = ix->w;
    if (!w.data) return fail(SPATTN_ERR_INVALID_ARG, "w: null data pointer");
    if (w.ndim != 3 || w.dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "w must be f32 [B, Nq, H_I]");
    if (w.shape[0] != q.shape[0] || w.shape[1] != q.shape[1] || w.shape[2] != H_I)
      return fail(SPATTN_ERR_INVALID_ARG, "w shape must be [B, Nq, H_I]");
    for (int i = 0; i < 3; ++i)
      if (w.stride[i] < 0) return fail(SPATTN_ERR_INVALID_ARG, "w: negative stride");
  }
  *B = q.shape[0];
  *Nq = q.shape[1];
  *ctx = k.shape[1];
  *G_sel = G;
  if (*Nq < 1 || *ctx < 1 || *Nq > *ctx) return fail(SPATTN_ERR_INVALID_ARG, "need 1 <= Nq <= ctx");
  return SPATTN_OK;
}

sp::IndexerParams indexer_params(const spattn_indexer* ix, const int32_t* ctx_len) {
  sp::IndexerParams p{};
  p.q = view(&ix->q_idx);
  p.k = view(&ix->k_idx);
  p.B = (int)ix->q_idx.shape[0];
  p.Nq = (int)ix->q_idx.shape[1];
  p.H_I = (int)ix->q_idx.shape[2];
  p.d_I = (int)ix->q_idx.shape[3];
  p.ctx = (int)ix->k_idx.shape[1];
  p.G_k = (int)ix->k_idx.shape[2];
  p.hpg = ix->heads_per_group;
  p.G_sel = p.H_I / p.hpg;
  p.relu = ix->score_mode == SPATTN_SCORE_WEIGHTED_RELU;
  if (p.relu) {
    p.w = (const float*)ix->w.data;
    for (int i = 0; i < 3; ++i) p.ws_[i] = ix->w.stride[i];
  }
  p.ctx_len = ctx_len;
  return p;
}

}  // namespace

extern "C" {

SPATTN_API const char* spattn_version(void) { return "libspattn 0.1.0 (gfx950)"; }

SPATTN_API const char* spattn_status_string(int status) {
  switch (status) {
    case SPATTN_OK: return "ok";
    case SPATTN_ERR_INVALID_ARG: return "invalid argument";
    case SPATTN_ERR_UNSUPPORTED: return "unsupported";
    case SPATTN_ERR_WORKSPACE: return "workspace too small";
    case SPATTN_ERR_NO_DEVICE: return "no usable device";
    case SPATTN_ERR_LAUNCH: return "launch failed";
  }
  return "unknown status";
}

SPATTN_API const char* spattn_last_error_message(void) { return g_err.c_str(); }

// ------------------------------------------------------------------ index scores
SPATTN_API size_t spattn_index_scores_workspace(const spattn_indexer* ix) {
  int64_t B, Nq, ctx, G;
  if (check_indexer(ix, &B, &Nq, &ctx, &G)) return (size_t)-1;
  return sp::indexer_ws_bytes((int)B, (int)ix->k_idx.shape[2], (int)ctx);
}

SPATTN_API int spattn_index_scores(const spattn_indexer* ix, const int32_t* ctx_len,
                                   const spattn_tensor* scores_out, float* err_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  int64_t B, Nq, ctx, G;
  int rc;
  if ((rc = check_indexer(ix, &B, &Nq, &ctx, &G))) return rc;
  if ((rc = check_tensor(scores_out, "scores_out", 4, false))) return rc;
  if (scores_out->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "scores_out must be f32");
  if (scores_out->shape[0] != B || scores_out->shape[1] != G || scores_out->shape[2] != Nq ||
      scores_out->shape[3] != ctx)
    return fail(SPATTN_ERR_INVALID_ARG, "scores_out must be [B, G_sel, Nq, ctx]");
  const size_t need = sp::indexer_ws_bytes((int)B, (int)ix->k_idx.shape[2], (int)ctx);
  if (ws_bytes < need || (need && !ws)) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if ((rc = device_ok())) return rc;
  sp::IndexerParams p = indexer_params(ix, ctx_len);
  p.scores = (float*)scores_out->data;
  for (int i = 0; i < 4; ++i) p.ss[i] = scores_out->stride[i];
  p.err = err_out;
  p.kmax = (float*)ws;
  return launched(sp::launch_index_scores(p, (hipStream_t)stream));
}

// ------------------------------------------------------------------ top-K
static int topk_setup(const spattn_tensor* scores, const float* err, const spattn_indexer* ix,
                      const int32_t* ctx_len, int32_t k, uint32_t flags, const spattn_tensor* idx_out,
                      sp::TopkParams& p) {
  int rc;
  p = sp::TopkParams{};
  if (flags & ~(SPATTN_TOPK_CERTIFIED | SPATTN_TOPK_FUSED_INDEX))
    return fail(SPATTN_ERR_INVALID_ARG, "unknown flags");
  if (k < 1 || k > 16384) return fail(SPATTN_ERR_INVALID_ARG, "k must be in 1..16384");
  int64_t B, G, Nq, ctx;
  if (flags & SPATTN_TOPK_FUSED_INDEX) {
    if (scores || err) return fail(SPATTN_ERR_INVALID_ARG, "fused selection takes no scores or err");
    if ((rc = check_indexer(ix, &B, &Nq, &ctx, &G))) return rc;
    p.certified = true;
    p.ix = indexer_params(ix, ctx_len);
  } else {
    if ((rc = check_tensor(scores, "scores", 4, false))) return rc;
    if (scores->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "scores must be f32");
    B = scores->shape[0];
    G = scores->shape[1];
    Nq = scores->shape[2];
    ctx = scores->shape[3];
    if (Nq < 1 || ctx < 1 || Nq > ctx) return fail(SPATTN_ERR_INVALID_ARG, "need 1 <= Nq <= ctx");
    if (flags & SPATTN_TOPK_CERTIFIED) {
      int64_t iB, iNq, ictx, iG;
      if (!err) return fail(SPATTN_ERR_INVALID_ARG, "certified selection needs err");
      if ((rc = check_indexer(ix, &iB, &iNq, &ictx, &iG))) return rc;
      if (iB != B || iNq != Nq || ictx != ctx || iG != G)
        return fail(SPATTN_ERR_INVALID_ARG, "indexer shapes do not match scores");
      p.certified = true;
      p.ix = indexer_params(ix, ctx_len);
    }
    p.scores = (const float*)scores->data;
    for (int i = 0; i < 4; ++i) p.ss[i] = scores->stride[i];
  }
  if (idx_out) {
    if ((rc = check_tensor(idx_out, "idx_out", 4, false))) return rc;
    if (idx_out->dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "idx_out must be int32");
    if (idx_out->shape[0] != B || idx_out->shape[1] != G || idx_out->shape[2] != Nq || idx_out->shape[3] != k)
      return fail(SPATTN_ERR_INVALID_ARG, "idx_out must be [B, G, Nq, k]");
    p.idx = (int32_t*)idx_out->data;
    for (int i = 0; i < 4; ++i) p.is[i] = idx_out->stride[i];
  }
  p.err = err;
  p.B = (int)B;
  p.G = (int)G;
  p.Nq = (int)Nq;
  p.ctx = (int)ctx;
  p.K = k;
  p.ctx_len = ctx_len;
  if ((flags & SPATTN_TOPK_FUSED_INDEX) && !sp::topk_fused_ok(p))
    return fail(SPATTN_ERR_UNSUPPORTED,
                "fused selection needs d_I = 64, bf16 q_idx, bf16/fp8 k_idx shared by all groups and either "
                "<= 4 heads per group, Nq * H_I <= 128 (power-of-two H_I), ctx <= 262144, or one group of "
                "4 weighted-ReLU heads with ctx <= 65536");
  return SPATTN_OK;
}

SPATTN_API size_t spattn_topk_workspace(const spattn_tensor* scores, const spattn_indexer* ix, int32_t k,
                                        uint32_t flags) {
  sp::TopkParams p;
  if (topk_setup(scores, nullptr, ix, nullptr, k, flags & ~SPATTN_TOPK_CERTIFIED, nullptr, p)) return (size_t)-1;
  return (flags & SPATTN_TOPK_FUSED_INDEX) ? sp::topk_fused_ws_bytes(p) : sp::topk_ws_bytes(p);
}

SPATTN_API int spattn_topk(const spattn_tensor* scores, const float* err, const spattn_indexer* ix,
                           const int32_t* ctx_len, int32_t k, uint32_t flags, const spattn_tensor* idx_out,
                           int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
  sp::TopkParams p;
  int rc;
  if (!idx_out) return fail(SPATTN_ERR_INVALID_ARG, "idx_out: null tensor");
  if ((rc = topk_setup(scores, err, ix, ctx_len, k, flags, idx_out, p))) return rc;
  p.count = count_out;
  const bool fused = (flags & SPATTN_TOPK_FUSED_INDEX) != 0;
  const size_t need = fused ? sp::topk_fused_ws_bytes(p) : sp::topk_ws_bytes(p);
  if (ws_bytes < need || (need && !ws)) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  p.ws = ws;
  if ((rc = device_ok())) return rc;
  return launched(fused ? sp::launch_topk_fused(p, (hipStream_t)stream) : sp::launch_topk(p, (hipStream_t)stream));
}

// ------------------------------------------------------------------ page select
static int log2_pow2(int32_t v, int32_t hi) {   // log2 of a power of two in 1..hi, else -1
  if (v < 1 || v > hi || (v & (v - 1))) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

static int page_select_setup(const spattn_tensor* scores, const float* err, const spattn_indexer* ix,
                             const int32_t* ctx_len, int32_t page_size, int32_t top_pages, int32_t n_local,
                             uint32_t flags, const spattn_tensor* pg_idx_out, sp::PageSelParams& q) {
  int rc;
  q = sp::PageSelParams{};
  if (flags & ~(SPATTN_TOPK_CERTIFIED | SPATTN_TOPK_FUSED_INDEX)) return fail(SPATTN_ERR_INVALID_ARG, "unknown flags");
  q.lgP = log2_pow2(page_size, 4096);
  if (q.lgP < 0) return fail(SPATTN_ERR_INVALID_ARG, "page_size must be a power of two in 1..4096");
  if (top_pages < 0 || n_local < 0 || (int64_t)top_pages + n_local < 1)
    return fail(SPATTN_ERR_INVALID_ARG, "need top_pages >= 0, n_local >= 0 and top_pages + n_local >= 1");
  if (top_pages > 16384 || n_local > 16384) return fail(SPATTN_ERR_UNSUPPORTED, "top_pages and n_local must be <= 16384");
  if (flags & SPATTN_TOPK_FUSED_INDEX) {
    if (scores || err) return fail(SPATTN_ERR_INVALID_ARG, "fused selection takes no scores or err");
    int64_t B, Nq, ctx, G;
    if ((rc = check_indexer(ix, &B, &Nq, &ctx, &G))) return rc;
    q.t.certified = true;
    q.t.ix = indexer_params(ix, ctx_len);
    q.t.B = (int)B;
    q.t.G = (int)G;
    q.t.Nq = (int)Nq;
    q.t.ctx = (int)ctx;
    q.t.ctx_len = ctx_len;
    q.fused = true;
  } else {
    if (!scores) return fail(SPATTN_ERR_INVALID_ARG, "scores: null tensor");
    if ((rc = topk_setup(scores, err, ix, ctx_len, 1, flags, nullptr, q.t))) return rc;
  }
  const int64_t npages = ((int64_t)q.t.ctx + page_size - 1) / page_size;
  if (npages > sp::kMaxPages) return fail(SPATTN_ERR_UNSUPPORTED, "more than %d pages per request", sp::kMaxPages);
  q.t.K = top_pages;
  q.n_local = n_local;
  q.width = top_pages + n_local;
  if (pg_idx_out) {
    if ((rc = check_tensor(pg_idx_out, "pg_idx_out", 4, false))) return rc;
    if (pg_idx_out->dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "pg_idx_out must be int32");
    if (pg_idx_out->shape[0] != q.t.B || pg_idx_out->shape[1] != q.t.G || pg_idx_out->shape[2] != q.t.Nq ||
        pg_idx_out->shape[3] != q.width)
      return fail(SPATTN_ERR_INVALID_ARG, "pg_idx_out must be [B, G, Nq, top_pages + n_local]");
    q.t.idx = (int32_t*)pg_idx_out->data;
    for (int i = 0; i < 4; ++i) q.t.is[i] = pg_idx_out->stride[i];
  }
  return SPATTN_OK;
}

SPATTN_API size_t spattn_page_select_workspace(const spattn_tensor* scores, const spattn_indexer* ix,
                                               int32_t page_size, int32_t top_pages, int32_t n_local,
                                               uint32_t flags) {
  sp::PageSelParams q;
  if (page_select_setup(scores, nullptr, ix, nullptr, page_size, top_pages, n_local,
                        flags & ~SPATTN_TOPK_CERTIFIED, nullptr, q))
    return (size_t)-1;
  return sp::page_select_ws_bytes(q);
}

SPATTN_API int spattn_page_select(const spattn_tensor* scores, const float* err, const spattn_indexer* ix,
                                  const int32_t* ctx_len, int32_t page_size, int32_t top_pages, int32_t n_local,
                                  uint32_t flags, const spattn_tensor* pg_idx_out, int32_t* pg_count_out, void* ws,
                                  size_t ws_bytes, void* stream) {
  sp::PageSelParams q;
  int rc;
  if (!pg_idx_out) return fail(SPATTN_ERR_INVALID_ARG, "pg_idx_out: null tensor");
  if ((rc = page_select_setup(scores, err, ix, ctx_len, page_size, top_pages, n_local, flags, pg_idx_out, q)))
    return rc;
  q.t.count = pg_count_out;
  const size_t need = sp::page_select_ws_bytes(q);
  if (ws_bytes < need || (need && !ws)) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  q.ws = ws;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_page_select(q, (hipStream_t)stream));
}

// ------------------------------------------------------------------ two-level selection
static int two_level_setup(const spattn_indexer* ix, const spattn_tensor* kp, const int32_t* ctx_len,
                           int32_t block_size, sp::TwoLevelParams& q) {
  int rc;
  q = sp::TwoLevelParams{};
  int64_t B, Nq, ctx, G;
  if ((rc = check_indexer(ix, &B, &Nq, &ctx, &G))) return rc;
  q.lgbs = log2_pow2(block_size, 4096);
  if (q.lgbs < 0) return fail(SPATTN_ERR_INVALID_ARG, "block_size must be a power of two in 1..4096");
  if ((ctx >> q.lgbs) > sp::kTlMaxCand) return fail(SPATTN_ERR_UNSUPPORTED, "more than %d blocks per request", sp::kTlMaxCand);
  if ((rc = check_tensor(kp, "k_blocks", 4, true))) return rc;
  if (kp->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "k_blocks must be f32");
  if (kp->shape[0] != B || kp->shape[1] < (ctx >> q.lgbs) || kp->shape[2] != ix->k_idx.shape[2] ||
      kp->shape[3] != ix->k_idx.shape[3])
    return fail(SPATTN_ERR_INVALID_ARG, "k_blocks must be [B, ctx / block_size, G_k, d_I]");
  q.t.ix = indexer_params(ix, ctx_len);
  q.t.certified = true;
  q.t.B = (int)B;
  q.t.G = (int)G;
  q.t.Nq = (int)Nq;
  q.t.ctx = (int)ctx;
  q.t.ctx_len = ctx_len;
  q.kp = (float*)kp->data;
  for (int i = 0; i < 4; ++i) q.kps[i] = kp->stride[i];
  return SPATTN_OK;
}

SPATTN_API int spattn_pool_index_keys(const spattn_indexer* ix, const int32_t* ctx_len, int32_t block_size,
                                      const spattn_tensor* k_blocks_out, void* stream) {
  sp::TwoLevelParams q;
  int rc;
  if ((rc = two_level_setup(ix, k_blocks_out, ctx_len, block_size, q))) return rc;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_pool_index_keys(q, (hipStream_t)stream));
}

SPATTN_API size_t spattn_topk_two_level_workspace(const spattn_indexer* ix, const spattn_tensor* k_blocks,
                                                  int32_t block_size, int32_t top_blocks, int32_t k) {
  sp::TwoLevelParams q;
  if (two_level_setup(ix, k_blocks, nullptr, block_size, q) || top_blocks < 1 || k < 1) return (size_t)-1;
  return 0;
}

SPATTN_API int spattn_topk_two_level(const spattn_indexer* ix, const spattn_tensor* k_blocks, const int32_t* ctx_len,
                                     int32_t block_size, int32_t top_blocks, int32_t k, const spattn_tensor* idx_out,
                                     int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
  sp::TwoLevelParams q;
  int rc;
  (void)ws;
  (void)ws_bytes;
  if ((rc = two_level_setup(ix, k_blocks, ctx_len, block_size, q))) return rc;
  if (top_blocks < 1 || k < 1 || k > 16384) return fail(SPATTN_ERR_INVALID_ARG, "need top_blocks >= 1 and 1 <= k <= 16384");
  if (((int64_t)top_blocks + 1) << q.lgbs > sp::kTlMaxCand)
    return fail(SPATTN_ERR_UNSUPPORTED, "(top_blocks + 1) * block_size must be <= %d", sp::kTlMaxCand);
  if ((rc = check_tensor(idx_out, "idx_out", 4, false))) return rc;
  if (idx_out->dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "idx_out must be int32");
  if (idx_out->shape[0] != q.t.B || idx_out->shape[1] != q.t.G || idx_out->shape[2] != q.t.Nq || idx_out->shape[3] != k)
    return fail(SPATTN_ERR_INVALID_ARG, "idx_out must be [B, G, Nq, k]");
  q.t.idx = (int32_t*)idx_out->data;
  for (int i = 0; i < 4; ++i) q.t.is[i] = idx_out->stride[i];
  q.t.count = count_out;
  q.t.K = k;
  q.nb = top_blocks;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_two_level(q, (hipStream_t)stream));
}

SPATTN_API int spattn_index_block_select(const spattn_indexer* ix, const spattn_tensor* k_blocks,
                                         const int32_t* ctx_len, int32_t block_size, int32_t top_blocks,
                                         const spattn_tensor* blk_idx_out, int32_t* blk_count_out, void* stream) {
  sp::TwoLevelParams q;
  int rc;
  if ((rc = two_level_setup(ix, k_blocks, ctx_len, block_size, q))) return rc;
  if (top_blocks < 1 || top_blocks > 16384) return fail(SPATTN_ERR_INVALID_ARG, "need 1 <= top_blocks <= 16384");
  if ((rc = check_tensor(blk_idx_out, "blk_idx_out", 4, false))) return rc;
  if (blk_idx_out->dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "blk_idx_out must be int32");
  if (blk_idx_out->shape[0] != q.t.B || blk_idx_out->shape[1] != q.t.G || blk_idx_out->shape[2] != q.t.Nq ||
      blk_idx_out->shape[3] != top_blocks)
    return fail(SPATTN_ERR_INVALID_ARG, "blk_idx_out must be [B, G, Nq, top_blocks]");
  q.t.idx = (int32_t*)blk_idx_out->data;
  for (int i = 0; i < 4; ++i) q.t.is[i] = blk_idx_out->stride[i];
  q.t.count = blk_count_out;
  q.t.K = top_blocks;
  q.nb = top_blocks;
  q.blocks_only = true;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_two_level(q, (hipStream_t)stream));
}

// ------------------------------------------------------------------ block select
static int check_qk(const spattn_tensor* q, const spattn_tensor* k) {
  int rc;
  if ((rc = check_tensor(q, "q", 4, true))) return rc;
  if ((rc = check_tensor(k, "k", 4, true))) return rc;
  if (q->dtype != k->dtype) return fail(SPATTN_ERR_INVALID_ARG, "q and k dtypes differ");
  if (q->dtype != SPATTN_F32 && q->dtype != SPATTN_BF16) return fail(SPATTN_ERR_UNSUPPORTED, "q/k dtype must be f32 or bf16");
  if (q->shape[0] != k->shape[0] || q->shape[3] != k->shape[3])
    return fail(SPATTN_ERR_INVALID_ARG, "q/k batch or head dim mismatch");
  if (k->shape[1] < 1 || q->shape[1] % k->shape[1])
    return fail(SPATTN_ERR_INVALID_ARG, "KV heads must divide query heads");
  if (q->shape[3] != 64 && q->shape[3] != 128) return fail(SPATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (q->shape[2] < 1 || q->shape[2] > k->shape[2]) return fail(SPATTN_ERR_INVALID_ARG, "need 1 <= Nq <= ctx");
  return SPATTN_OK;
}

SPATTN_API size_t spattn_block_select_workspace(const spattn_tensor* q, const spattn_tensor* k,
                                                int32_t block_size, int32_t top_blocks) {
  if (check_qk(q, k) || block_size < 1 || top_blocks < 1) return (size_t)-1;
  return sp::block_select_ws_bytes((int)k->shape[0], (int)k->shape[1], (int)k->shape[2], (int)k->shape[3], block_size);
}

SPATTN_API int spattn_block_select(const spattn_tensor* q, const spattn_tensor* k, const int32_t* ctx_len,
                                   int32_t block_size, int32_t top_blocks, const spattn_tensor* blk_idx_out,
                                   int32_t* blk_count_out, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_qk(q, k))) return rc;
  if (block_size < 1 || (block_size & (block_size - 1)))
    return fail(SPATTN_ERR_INVALID_ARG, "block_size must be a power of two");
  if (top_blocks < 1) return fail(SPATTN_ERR_INVALID_ARG, "top_blocks must be >= 1");
  if (k->shape[2] / block_size > 2048) return fail(SPATTN_ERR_UNSUPPORTED, "more than 2048 blocks per request");
  if ((rc = check_tensor(blk_idx_out, "blk_idx_out", 4, false))) return rc;
  if (blk_idx_out->dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "blk_idx_out must be int32");
  if (blk_idx_out->shape[0] != q->shape[0] || blk_idx_out->shape[1] != q->shape[1] ||
      blk_idx_out->shape[2] != q->shape[2] || blk_idx_out->shape[3] != top_blocks)
    return fail(SPATTN_ERR_INVALID_ARG, "blk_idx_out must be [B, H_q, Nq, top_blocks]");
  const size_t need = sp::block_select_ws_bytes((int)k->shape[0], (int)k->shape[1], (int)k->shape[2],
                                                (int)k->shape[3], block_size);
  if (ws_bytes < need || !ws) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if ((rc = device_ok())) return rc;
  sp::BlockSelectParams p{};
  p.q = view(q);
  p.k = view(k);
  p.B = (int)q->shape[0];
  p.Hq = (int)q->shape[1];
  p.Nq = (int)q->shape[2];
  p.d = (int)q->shape[3];
  p.Hkv = (int)k->shape[1];
  p.ctx = (int)k->shape[2];
  p.bs = block_size;
  p.log2bs = __builtin_ctz((unsigned)block_size);
  p.nb = top_blocks;
  p.ctx_len = ctx_len;
  p.out = (int32_t*)blk_idx_out->data;
  for (int i = 0; i < 4; ++i) p.os[i] = blk_idx_out->stride[i];
  p.count = blk_count_out;
  const size_t nbk = p.ctx / p.bs;
  const size_t nblk = (size_t)p.B * p.Hkv * nbk;
  p.kbar64 = (double*)ws;                                 // 8-byte aligned first
  p.kbar = (float*)(p.kbar64 + nblk * p.d);
  p.kabs = p.kbar + nblk * p.d;
  p.kexact = (uint32_t*)(p.kabs + nblk);
  const uintptr_t kb2 = ((uintptr_t)(p.kexact + nblk) + 255) & ~(uintptr_t)255;
  p.kb2 = (uint16_t*)kb2;
  return launched(sp::launch_block_select(p, (hipStream_t)stream));
}

// ------------------------------------------------------------------ attention
// q [B, H_q, Nq, d] against a page pool [n_pages, H_kv, P, d] and its table
static int check_q_pool(const spattn_tensor* q, const spattn_tensor* k, const spattn_kv_pages* pg, int& lgP,
                        int64_t& ctx) {
  int rc;
  if ((rc = check_tensor(q, "q", 4, true))) return rc;
  if ((rc = check_tensor(k, "k_pool", 4, true))) return rc;
  if (q->dtype != k->dtype) return fail(SPATTN_ERR_INVALID_ARG, "q and k_pool dtypes differ");
  if (q->dtype != SPATTN_F32 && q->dtype != SPATTN_BF16)
    return fail(SPATTN_ERR_UNSUPPORTED, "q/k dtype must be f32 or bf16");
  if (q->shape[3] != k->shape[3]) return fail(SPATTN_ERR_INVALID_ARG, "q/k_pool head dim mismatch");
  if (k->shape[1] < 1 || q->shape[1] % k->shape[1])
    return fail(SPATTN_ERR_INVALID_ARG, "KV heads must divide query heads");
  if (q->shape[3] != 64 && q->shape[3] != 128) return fail(SPATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  lgP = log2_pow2(pg->page_size, 4096);
  if (lgP < 0) return fail(SPATTN_ERR_INVALID_ARG, "page_size must be a power of two in 1..4096");
  if (k->shape[2] != pg->page_size) return fail(SPATTN_ERR_INVALID_ARG, "k_pool must be [n_pages, H_kv, page_size, d]");
  if (k->shape[0] < 1 || k->shape[0] * (int64_t)pg->page_size >= ((int64_t)1 << 31))
    return fail(SPATTN_ERR_UNSUPPORTED, "need 1 <= n_pages and n_pages * page_size < 2^31");
  if ((rc = check_tensor(&pg->page_table, "page_table", 2, false))) return rc;
  if (pg->page_table.dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "page_table must be int32");
  if (pg->page_table.shape[0] != q->shape[0] || pg->page_table.shape[1] < 1)
    return fail(SPATTN_ERR_INVALID_ARG, "page_table must be [B, max_pages]");
  ctx = pg->page_table.shape[1] * (int64_t)pg->page_size;
  if (ctx >= ((int64_t)1 << 31)) return fail(SPATTN_ERR_UNSUPPORTED, "max_pages * page_size must be < 2^31");
  if (q->shape[2] < 1 || q->shape[2] > ctx) return fail(SPATTN_ERR_INVALID_ARG, "need 1 <= Nq <= ctx");
  return SPATTN_OK;
}

static int attn_setup(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                      const spattn_selection* sel, sp::AttnParams& p, bool need_v,
                      const spattn_kv_pages* pages = nullptr) {
  int rc;
  int lgP = 0;
  int64_t pctx = 0;
  if (pages) {
    if ((rc = check_q_pool(q, k, pages, lgP, pctx))) return rc;
  } else if ((rc = check_qk(q, k))) {
    return rc;
  }
  if (need_v) {
    if ((rc = check_tensor(v, "v", 4, true))) return rc;
    if (v->dtype != k->dtype) return fail(SPATTN_ERR_INVALID_ARG, "v dtype differs from k");
    for (int i = 0; i < 4; ++i)
      if (v->shape[i] != k->shape[i]) return fail(SPATTN_ERR_INVALID_ARG, "v shape differs from k");
  }
  if (!sel) return fail(SPATTN_ERR_INVALID_ARG, "selection: null");
  p = sp::AttnParams{};
  p.q = view(q);
  p.k = view(k);
  if (need_v) p.v = view(v);
  p.B = (int)q->shape[0];
  p.Hq = (int)q->shape[1];
  p.Nq = (int)q->shape[2];
  p.d = (int)q->shape[3];
  p.Hkv = (int)k->shape[1];
  p.ctx = pages ? (int)pctx : (int)k->shape[2];
  if (pages) {
    p.ptab = (const int32_t*)pages->page_table.data;
    p.pts = pages->page_table.stride[0];
    p.lgP = lgP;
  }
  p.mode = sel->mode;
  p.G_sel = 1;
  switch (sel->mode) {
    case SPATTN_SEL_DENSE: break;
    case SPATTN_SEL_INDEX: {
      if ((rc = check_tensor(&sel->idx, "sel.idx", 4, false))) return rc;
      if (sel->idx.dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "sel.idx must be int32");
      const int64_t G = sel->idx.shape[1];
      if (sel->idx.shape[0] != p.B || sel->idx.shape[2] != p.Nq || G < 1 || p.Hq % G)
        return fail(SPATTN_ERR_INVALID_ARG, "sel.idx must be [B, G_sel, Nq, K] with G_sel | H_q");
      if ((G % p.Hkv) && (p.Hkv % G))
        return fail(SPATTN_ERR_INVALID_ARG, "G_sel and H_kv must divide one another");
      p.G_sel = (int)G;
      p.K = (int)sel->idx.shape[3];
      p.sel = (const int32_t*)sel->idx.data;
      for (int i = 0; i < 4; ++i) p.sels[i] = sel->idx.stride[i];
      break;
    }
    case SPATTN_SEL_WINDOW_GLOBAL:
      if (sel->window < 0 || sel->n_global < 0) return fail(SPATTN_ERR_INVALID_ARG, "window/n_global must be >= 0");
      if (sel->stride < 0 || sel->stride > (1 << 24))
        return fail(SPATTN_ERR_INVALID_ARG, "stride must be in 0..2^24");
      p.window = sel->window;
      p.n_global = sel->n_global;
      p.stride = sel->stride;
      break;
    case SPATTN_SEL_BLOCKS: {
      if ((rc = check_tensor(&sel->idx, "sel.idx", 4, false))) return rc;
      if (sel->idx.dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "sel.idx must be int32");
      if (sel->idx.shape[0] != p.B || sel->idx.shape[1] < 1 || p.Hq % sel->idx.shape[1] || sel->idx.shape[2] != p.Nq)
        return fail(SPATTN_ERR_INVALID_ARG, "block list must be [B, G_sel, Nq, nb] with G_sel | H_q");
      if (sel->block_size < 1 || sel->window < 0) return fail(SPATTN_ERR_INVALID_ARG, "bad block_size/window");
      p.G_sel = (int)sel->idx.shape[1];
      p.K = (int)sel->idx.shape[3];
      p.sel = (const int32_t*)sel->idx.data;
      for (int i = 0; i < 4; ++i) p.sels[i] = sel->idx.stride[i];
      p.bs = sel->block_size;
      p.window = sel->window;
      break;
    }
    case SPATTN_SEL_PAGES: {
      if ((rc = check_tensor(&sel->idx, "sel.idx", 4, false))) return rc;
      if (sel->idx.dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "sel.idx must be int32");
      const int64_t G = sel->idx.shape[1];
      if (sel->idx.shape[0] != p.B || sel->idx.shape[2] != p.Nq || G < 1 || p.Hq % G)
        return fail(SPATTN_ERR_INVALID_ARG, "page list must be [B, G_sel, Nq, np] with G_sel | H_q");
      if ((G % p.Hkv) && (p.Hkv % G))
        return fail(SPATTN_ERR_INVALID_ARG, "G_sel and H_kv must divide one another");
      const int lg = log2_pow2(sel->block_size, 4096);
      if (lg < 0) return fail(SPATTN_ERR_INVALID_ARG, "PAGES: block_size must be a power of two in 1..4096");
      const int64_t slots = sel->idx.shape[3] << lg;
      if (slots >= ((int64_t)1 << 31)) return fail(SPATTN_ERR_UNSUPPORTED, "page list covers too many tokens");
      p.G_sel = (int)G;
      p.K = (int)slots;
      p.bs = sel->block_size;
      p.lgbs = lg;
      p.sel = (const int32_t*)sel->idx.data;
      for (int i = 0; i < 4; ++i) p.sels[i] = sel->idx.stride[i];
      break;
    }
    default: return fail(SPATTN_ERR_INVALID_ARG, "unknown selection mode %d", sel->mode);
  }
  return SPATTN_OK;
}

SPATTN_API size_t spattn_sparse_attn_bwd_workspace(const spattn_tensor* q, const spattn_tensor* k,
                                                   const spattn_selection* sel) {
  sp::AttnParams p;
  if (attn_setup(q, k, nullptr, sel, p, false)) return (size_t)-1;
  return sp::attn_bwd_ws_bytes(p);
}

SPATTN_API size_t spattn_sparse_attn_fwd_workspace(const spattn_tensor* q, const spattn_tensor* k,
                                                   const spattn_selection* sel) {
  sp::AttnParams p;
  if (attn_setup(q, k, nullptr, sel, p, false)) return (size_t)-1;
  return sp::attn_ws_bytes(p);
}

}  // extern "C"

namespace spapi {

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

int device_check() { return device_ok(); }

int attn_fwd_prepare(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                     const spattn_kv_pages* pages, const int32_t* ctx_len, float scale, const spattn_selection* sel,
                     const spattn_tensor* o_out, float* lse_out, sp::AttnParams& p, size_t& need) {
  int rc;
  if ((rc = attn_setup(q, k, v, sel, p, true, pages))) return rc;
  if ((rc = check_tensor(o_out, "o_out", 4, false))) return rc;
  if (o_out->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "o_out must be f32");
  for (int i = 0; i < 4; ++i)
    if (o_out->shape[i] != q->shape[i]) return fail(SPATTN_ERR_INVALID_ARG, "o_out shape must equal q's");
  if (!(scale >= 0.f) || std::isinf(scale)) return fail(SPATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  p.scale = scale == 0.f ? 1.0f / std::sqrt((float)p.d) : scale;
  p.ctx_len = ctx_len;
  p.o = (float*)o_out->data;
  for (int i = 0; i < 4; ++i) p.os[i] = o_out->stride[i];
  p.lse = lse_out;
  need = sp::attn_ws_bytes(p);
  return SPATTN_OK;
}

int attn_fwd_launch(sp::AttnParams& p, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  p.ws = ws;
  p.ws_bytes = ws_bytes;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_attention(p, (hipStream_t)stream));
}

}  // namespace spapi

extern "C" {

static int attn_fwd(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                    const spattn_kv_pages* pages, const int32_t* ctx_len, float scale, const spattn_selection* sel,
                    const spattn_tensor* o_out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  sp::AttnParams p;
  size_t need = 0;
  int rc;
  if ((rc = spapi::attn_fwd_prepare(q, k, v, pages, ctx_len, scale, sel, o_out, lse_out, p, need))) return rc;
  if (ws_bytes < need || (need && !ws)) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  return spapi::attn_fwd_launch(p, ws, ws_bytes, stream);
}

SPATTN_API int spattn_sparse_attn_fwd(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                                      const int32_t* ctx_len, float scale, const spattn_selection* sel,
                                      const spattn_tensor* o_out, float* lse_out, void* ws, size_t ws_bytes,
                                      void* stream) {
  return attn_fwd(q, k, v, nullptr, ctx_len, scale, sel, o_out, lse_out, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ backward
static int check_f32_like(const spattn_tensor* t, const char* name, const int64_t* shape) {
  int rc;
  if ((rc = check_tensor(t, name, 4, false))) return rc;
  if (t->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "%s must be f32", name);
  for (int i = 0; i < 4; ++i)
    if (t->shape[i] != shape[i]) return fail(SPATTN_ERR_INVALID_ARG, "%s has the wrong shape", name);
  return SPATTN_OK;
}

SPATTN_API int spattn_sparse_attn_bwd(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                                      const int32_t* ctx_len, float scale, const spattn_selection* sel,
                                      const spattn_tensor* o, const float* lse, const spattn_tensor* d_o,
                                      const spattn_tensor* dq_out, const spattn_tensor* dk_out,
                                      const spattn_tensor* dv_out, void* ws, size_t ws_bytes, void* stream) {
  sp::AttnParams p;
  sp::AttnBwd g{};
  int rc;
  if ((rc = attn_setup(q, k, v, sel, p, true))) return rc;
  if (!lse) return fail(SPATTN_ERR_INVALID_ARG, "lse: null (the forward's LSE is required)");
  if ((rc = check_f32_like(o, "o", q->shape))) return rc;
  if ((rc = check_f32_like(d_o, "d_o", q->shape))) return rc;
  if ((rc = check_f32_like(dq_out, "dq_out", q->shape))) return rc;
  if ((rc = check_f32_like(dk_out, "dk_out", k->shape))) return rc;
  if ((rc = check_f32_like(dv_out, "dv_out", k->shape))) return rc;
  if (!(scale >= 0.f) || std::isinf(scale)) return fail(SPATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  p.scale = scale == 0.f ? 1.0f / std::sqrt((float)p.d) : scale;
  p.ctx_len = ctx_len;
  g.o = (const float*)o->data;
  g.lse = lse;
  g.dO = (const float*)d_o->data;
  g.dq = (float*)dq_out->data;
  g.dk = (float*)dk_out->data;
  g.dv = (float*)dv_out->data;
  const size_t need = sp::attn_bwd_ws_bytes(p);
  if (ws_bytes < need || (need && !ws)) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  g.part = need ? (float*)ws : nullptr;
  g.nslot = need ? sp::attn_bwd_slots(p) : 0;
  for (int i = 0; i < 4; ++i) {
    g.os[i] = o->stride[i];
    g.dos[i] = d_o->stride[i];
    g.dqs[i] = dq_out->stride[i];
    g.dks[i] = dk_out->stride[i];
    g.dvs[i] = dv_out->stride[i];
  }
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_attention_bwd(p, g, (hipStream_t)stream));
}

// ------------------------------------------------------------------ NSA
static int nsa_setup(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v, int32_t block_size,
                     const spattn_tensor* blk_idx, int32_t window, sp::NsaParams& p, bool need_v) {
  int rc;
  p = sp::NsaParams{};
  if (!blk_idx) return fail(SPATTN_ERR_INVALID_ARG, "blk_idx: null tensor");
  if (log2_pow2(block_size, 4096) < 0) return fail(SPATTN_ERR_INVALID_ARG, "block_size must be a power of two in 1..4096");
  if (window < 0) return fail(SPATTN_ERR_INVALID_ARG, "window must be >= 0");
  spattn_selection sel{};
  sel.mode = SPATTN_SEL_BLOCKS;
  sel.idx = *blk_idx;
  sel.block_size = block_size;
  if ((rc = attn_setup(q, k, v, &sel, p.a, need_v))) return rc;
  if (p.a.G_sel != p.a.Hq) return fail(SPATTN_ERR_INVALID_ARG, "blk_idx must be [B, H_q, Nq, nb]");
  p.a.window = window;
  return SPATTN_OK;
}

SPATTN_API size_t spattn_nsa_fwd_workspace(const spattn_tensor* q, const spattn_tensor* k, int32_t block_size,
                                           const spattn_tensor* blk_idx, int32_t window) {
  sp::NsaParams p;
  if (nsa_setup(q, k, nullptr, block_size, blk_idx, window, p, false)) return (size_t)-1;
  return sp::nsa_ws_bytes(p);
}

SPATTN_API int spattn_nsa_fwd(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                              const int32_t* ctx_len, float scale, int32_t block_size, const spattn_tensor* blk_idx,
                              int32_t window, const spattn_tensor* gates, const spattn_tensor* o_out, void* ws,
                              size_t ws_bytes, void* stream) {
  sp::NsaParams p;
  int rc;
  if ((rc = nsa_setup(q, k, v, block_size, blk_idx, window, p, true))) return rc;
  if ((rc = check_tensor(gates, "gates", 4, false))) return rc;
  if (gates->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "gates must be f32");
  if (gates->shape[0] != q->shape[0] || gates->shape[1] != q->shape[1] || gates->shape[2] != q->shape[2] ||
      gates->shape[3] != 3)
    return fail(SPATTN_ERR_INVALID_ARG, "gates must be [B, H_q, Nq, 3]");
  if ((rc = check_tensor(o_out, "o_out", 4, false))) return rc;
  if (o_out->dtype != SPATTN_F32) return fail(SPATTN_ERR_INVALID_ARG, "o_out must be f32");
  for (int i = 0; i < 4; ++i)
    if (o_out->shape[i] != q->shape[i]) return fail(SPATTN_ERR_INVALID_ARG, "o_out shape must equal q's");
  if (!(scale >= 0.f) || std::isinf(scale)) return fail(SPATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  p.a.scale = scale == 0.f ? 1.0f / std::sqrt((float)p.a.d) : scale;
  p.a.ctx_len = ctx_len;
  p.gates = (const float*)gates->data;
  for (int i = 0; i < 4; ++i) p.gs[i] = gates->stride[i];
  p.o = (float*)o_out->data;
  for (int i = 0; i < 4; ++i) p.os[i] = o_out->stride[i];
  const size_t need = sp::nsa_ws_bytes(p);
  if (ws_bytes < need || !ws) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  p.ws = ws;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_nsa(p, (hipStream_t)stream));
}

SPATTN_API size_t spattn_sparse_attn_fwd_paged_workspace(const spattn_tensor* q, const spattn_tensor* k_pool,
                                                         const spattn_kv_pages* pages, const spattn_selection* sel) {
  sp::AttnParams p;
  if (!pages || attn_setup(q, k_pool, nullptr, sel, p, false, pages)) return (size_t)-1;
  return sp::attn_ws_bytes(p);
}

SPATTN_API int spattn_sparse_attn_fwd_paged(const spattn_tensor* q, const spattn_tensor* k_pool,
                                            const spattn_tensor* v_pool, const spattn_kv_pages* pages,
                                            const int32_t* ctx_len, float scale, const spattn_selection* sel,
                                            const spattn_tensor* o_out, float* lse_out, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (!pages) return fail(SPATTN_ERR_INVALID_ARG, "pages: null");
  return attn_fwd(q, k_pool, v_pool, pages, ctx_len, scale, sel, o_out, lse_out, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ Quest page selection
static int check_bounds(const spattn_tensor* bnd, int64_t B, int64_t Hkv, int64_t d, int dt, int64_t& maxp) {
  int rc;
  if ((rc = check_tensor(bnd, "bounds", 4, true))) return rc;
  if (bnd->dtype != dt) return fail(SPATTN_ERR_INVALID_ARG, "bounds must have the key dtype");
  if (bnd->shape[0] != B || bnd->shape[2] != Hkv || bnd->shape[3] != 2 * d || bnd->shape[1] < 1)
    return fail(SPATTN_ERR_INVALID_ARG, "bounds must be [B, max_pages, H_kv, 2d]");
  maxp = bnd->shape[1];
  return SPATTN_OK;
}

SPATTN_API int spattn_quest_page_bounds(const spattn_tensor* k_pool, const spattn_kv_pages* pages,
                                        const int32_t* ctx_len, const spattn_tensor* bounds_out, void* stream) {
  int rc;
  if (!pages) return fail(SPATTN_ERR_INVALID_ARG, "pages: null");
  if ((rc = check_tensor(k_pool, "k_pool", 4, true))) return rc;
  if (k_pool->dtype != SPATTN_F32 && k_pool->dtype != SPATTN_BF16)
    return fail(SPATTN_ERR_UNSUPPORTED, "k_pool dtype must be f32 or bf16");
  const int64_t Hkv = k_pool->shape[1], d = k_pool->shape[3];
  if (d != 64 && d != 128) return fail(SPATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  const int lgP = log2_pow2(pages->page_size, 4096);
  if (lgP < 0) return fail(SPATTN_ERR_INVALID_ARG, "page_size must be a power of two in 1..4096");
  if (k_pool->shape[2] != pages->page_size || Hkv < 1 || k_pool->shape[0] < 1)
    return fail(SPATTN_ERR_INVALID_ARG, "k_pool must be [n_pages, H_kv, page_size, d]");
  if ((rc = check_tensor(&pages->page_table, "page_table", 2, false))) return rc;
  if (pages->page_table.dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "page_table must be int32");
  const int64_t B = pages->page_table.shape[0], tabp = pages->page_table.shape[1];
  if (B < 1 || tabp < 1) return fail(SPATTN_ERR_INVALID_ARG, "page_table must be [B, max_pages]");
  int64_t maxp;
  if ((rc = check_bounds(bounds_out, B, Hkv, d, k_pool->dtype, maxp))) return rc;
  if (maxp != tabp) return fail(SPATTN_ERR_INVALID_ARG, "bounds and page_table disagree on max_pages");
  if (maxp * pages->page_size >= ((int64_t)1 << 31) || maxp > 65535)
    return fail(SPATTN_ERR_UNSUPPORTED, "max_pages too large");
  sp::QuestParams p{};
  p.kp = view(k_pool);
  p.ptab = (const int32_t*)pages->page_table.data;
  p.pts[0] = pages->page_table.stride[0];
  p.pts[1] = pages->page_table.stride[1];
  p.bnd = bounds_out->data;
  for (int i = 0; i < 3; ++i) p.bs[i] = bounds_out->stride[i];
  p.B = (int)B;
  p.Hkv = (int)Hkv;
  p.d = (int)d;
  p.dt = k_pool->dtype;
  p.lgP = lgP;
  p.maxp = (int)maxp;
  p.ctx = (int)(maxp << lgP);
  p.ctx_len = ctx_len;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_quest_bounds(p, (hipStream_t)stream));
}

static int quest_setup(const spattn_tensor* q, const spattn_tensor* bounds, const int32_t* ctx_len,
                       int32_t page_size, int32_t top_pages, int32_t n_local, const spattn_tensor* pg_idx_out,
                       sp::QuestParams& p) {
  int rc;
  p = sp::QuestParams{};
  if ((rc = check_tensor(q, "q", 4, true))) return rc;
  if (q->dtype != SPATTN_F32 && q->dtype != SPATTN_BF16) return fail(SPATTN_ERR_UNSUPPORTED, "q dtype must be f32 or bf16");
  const int64_t B = q->shape[0], Hq = q->shape[1], Nq = q->shape[2], d = q->shape[3];
  if (d != 64 && d != 128) return fail(SPATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (!bounds) return fail(SPATTN_ERR_INVALID_ARG, "bounds: null tensor");
  const int64_t Hkv = bounds->ndim == 4 ? bounds->shape[2] : 0;
  if (Hkv < 1 || Hq % Hkv) return fail(SPATTN_ERR_INVALID_ARG, "KV heads must divide query heads");
  int64_t maxp;
  if ((rc = check_bounds(bounds, B, Hkv, d, q->dtype, maxp))) return rc;
  const int lgP = log2_pow2(page_size, 4096);
  if (lgP < 0) return fail(SPATTN_ERR_INVALID_ARG, "page_size must be a power of two in 1..4096");
  if (maxp > sp::kMaxPages) return fail(SPATTN_ERR_UNSUPPORTED, "more than %d pages per request", sp::kMaxPages);
  const int64_t ctx = maxp << lgP;
  if (ctx >= ((int64_t)1 << 31)) return fail(SPATTN_ERR_UNSUPPORTED, "max_pages * page_size must be < 2^31");
  if (Nq < 1 || Nq > ctx) return fail(SPATTN_ERR_INVALID_ARG, "need 1 <= Nq <= ctx");
  if (top_pages < 0 || top_pages > 16384) return fail(SPATTN_ERR_INVALID_ARG, "top_pages must be in 0..16384");
  if (n_local < 1 || n_local > 16384)
    return fail(SPATTN_ERR_INVALID_ARG, "n_local must be in 1..16384 (the page holding the query is always read)");
  if (!pg_idx_out) return fail(SPATTN_ERR_INVALID_ARG, "pg_idx_out: null tensor");
  if ((rc = check_tensor(pg_idx_out, "pg_idx_out", 4, false))) return rc;
  if (pg_idx_out->dtype != SPATTN_I32) return fail(SPATTN_ERR_INVALID_ARG, "pg_idx_out must be int32");
  const int64_t G = pg_idx_out->shape[1];
  if (pg_idx_out->shape[0] != B || pg_idx_out->shape[2] != Nq || pg_idx_out->shape[3] != (int64_t)top_pages + n_local)
    return fail(SPATTN_ERR_INVALID_ARG, "pg_idx_out must be [B, G, Nq, top_pages + n_local]");
  if (G < 1 || G % Hkv || Hq % G) return fail(SPATTN_ERR_INVALID_ARG, "selection groups G: H_kv | G | H_q");
  if (Hq / G > 16) return fail(SPATTN_ERR_UNSUPPORTED, "at most 16 query heads per selection group");
  if (B * G * Nq > 65535) return fail(SPATTN_ERR_UNSUPPORTED, "B * G * Nq must be <= 65535");
  p.q = view(q);
  p.bnd = bounds->data;
  for (int i = 0; i < 3; ++i) p.bs[i] = bounds->stride[i];
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.d = (int)d;
  p.dt = q->dtype;
  p.lgP = lgP;
  p.maxp = (int)maxp;
  p.ctx = (int)ctx;
  p.ctx_len = ctx_len;
  sp::PageSelParams& s = p.sel;
  s.t.B = (int)B;
  s.t.G = (int)G;
  s.t.Nq = (int)Nq;
  s.t.ctx = (int)ctx;
  s.t.K = top_pages;
  s.t.ctx_len = ctx_len;
  s.t.certified = false;
  s.t.idx = (int32_t*)pg_idx_out->data;
  for (int i = 0; i < 4; ++i) s.t.is[i] = pg_idx_out->stride[i];
  s.lgP = lgP;
  s.n_local = n_local;
  s.width = top_pages + n_local;
  return SPATTN_OK;
}

SPATTN_API size_t spattn_quest_select_workspace(const spattn_tensor* q, const spattn_tensor* bounds,
                                                int32_t page_size, int32_t top_pages, int32_t n_local,
                                                const spattn_tensor* pg_idx_out) {
  sp::QuestParams p;
  if (quest_setup(q, bounds, nullptr, page_size, top_pages, n_local, pg_idx_out, p)) return (size_t)-1;
  return sp::quest_ws_bytes(p);
}

SPATTN_API int spattn_quest_select(const spattn_tensor* q, const spattn_tensor* bounds, const int32_t* ctx_len,
                                   int32_t page_size, int32_t top_pages, int32_t n_local,
                                   const spattn_tensor* pg_idx_out, int32_t* pg_count_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  sp::QuestParams p;
  int rc;
  if ((rc = quest_setup(q, bounds, ctx_len, page_size, top_pages, n_local, pg_idx_out, p))) return rc;
  p.sel.t.count = pg_count_out;
  const size_t need = sp::quest_ws_bytes(p);
  if (ws_bytes < need || (need && !ws)) return fail(SPATTN_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  p.sel.ws = ws;
  if ((rc = device_ok())) return rc;
  return launched(sp::launch_quest_select(p, (hipStream_t)stream));
}

}  // extern "C"
