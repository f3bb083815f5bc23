// Page-granular selection ("Sparse Attention in 2026: Why It Finally Had to Be
// Native", DSA list: the indexer rates every KV page, attention reads the
// best pages plus the mandatory recent pages, whole).
//
// Row (b, g, r) at position p: page pg holds tokens pg*P .. pg*P+P-1. The
// n_local pages ending with page p/P are always read; every earlier page is a
// candidate whose key is the largest key among its tokens (within 0..p), and
// the top_pages candidates largest by (key descending, page ascending) join
// them. The list is written ascending.
//
// One 512-thread workgroup per row:
//  1. page keys: the row's scores are read once, coalesced (four tokens per
//     lane when the row is 16-byte aligned), and folded per page by lane
//     shuffles; pages wider than a wave's sweep are merged by LDS atomics.
//     Keys stay in LDS (up to kMaxPages candidates). With few rows (decode)
//     this pass is spread over many workgroups per row instead (page_keys
//     kernel, kPkChunk tokens each), which leave the keys in the workspace;
//     in the fused call the MFMA indexer writes them from its epilogue.
//  2. radix select of the top_pages-th largest page key t.
//  3. uncertified: pages above t are in, pages equal to t go in by index.
//     Certified (scores within eps of the exact keys): pages whose computed key
//     is above t + 2 eps are in the exact selection and pages below t - 2 eps
//     are out. A band page's exact key is the largest exact key among its
//     tokens, and only tokens whose computed score reaches the page's computed
//     key - 2 eps can hold it (any other token's exact key lies below the
//     exact key of the page's best computed token). Those tokens are rescored
//     exactly, and the remaining slots go to the band's best by (exact key
//     descending, page ascending).
#include "common.h"
#include "exact.h"
#include "internal.h"
#include "rowselect.h"

namespace sp {

constexpr int kPsThreads = 512;
constexpr int kPsBandCap = 2048;
constexpr int kPkThreads = 256;
constexpr int kPkChunk = 8192;      // tokens per page-key workgroup (a multiple of every page size)
constexpr int kPsFewRows = 512;     // up to this many rows the page keys get their own kernel

struct PsSmem {
  uint32_t pk[kMaxPages];        // order keys of the candidate pages
  uint32_t hist[4096];
  uint32_t band_j[kPsBandCap];
  uint32_t band_k[kPsBandCap];
  uint32_t sc[16];
  uint32_t run[4];
  float red[32];
};

// Keys of pages 0..npc-1 from the scores of tokens 0..ntok-1 (ntok covers the
// candidate pages, cut at p); pk is zeroed first (0 is below every float key).
template <int T>
SP_DEV void page_keys(const float* s, int ntok, int lgP, int npc, uint32_t* pk) {
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < npc; i += T) pk[i] = 0u;
  __syncthreads();
  const bool vec = lgP >= 2 && (((uintptr_t)s) & 15) == 0;
  const int lg_per = vec ? 2 : 0;                 // log2 tokens per lane
  const int lgG = lgP - lg_per;                   // log2 lanes per page
  const int lim = lgG < 6 ? lgG : 6;              // shuffle steps inside a wave
  const bool whole = lgG <= 6;                    // one lane group holds the whole page
  constexpr int U = 4;
  const int step = T << lg_per;                   // tokens per sweep of the workgroup
  for (int base = 0; base < ntok; base += step * U) {
    uint32_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t0 = base + u * step + (tid << lg_per);
      if (vec) {
        if (t0 + 3 < ntok) {
          const f32x4 v = *(const f32x4*)(s + t0);
          m[u] = max(max(f32_order_key(v[0]), f32_order_key(v[1])), max(f32_order_key(v[2]), f32_order_key(v[3])));
        } else {
          uint32_t mm = 0u;
          for (int e = 0; e < 4; ++e)
            if (t0 + e < ntok) mm = max(mm, f32_order_key(s[t0 + e]));
          m[u] = mm;
        }
      } else {
        m[u] = t0 < ntok ? f32_order_key(s[t0]) : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t0 = base + u * step + (tid << lg_per);
      uint32_t v = m[u];
      for (int o = 0; o < lim; ++o) v = max(v, (uint32_t)__shfl_xor((int)v, 1 << o, 64));
      const int page = t0 >> lgP;
      if ((lane & ((1 << lim) - 1)) == 0 && page < npc) {
        if (whole) pk[page] = v;
        else atomicMax(&pk[page], v);
      }
    }
  }
  __syncthreads();
}

// Keys of the candidate pages of one row in the token range of one
// workgroup, written to pkg[row * npmax + page].
__global__ __launch_bounds__(kPkThreads) void page_keys_kernel(PageSelParams q, uint32_t* pkg, int npmax) {
  __shared__ uint32_t pk[kPkChunk];
  const TopkParams& p = q.t;
  const int row = blockIdx.y;
  const int r = row % p.Nq, g = (row / p.Nq) % p.G, b = row / (p.Nq * p.G);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  if (pos < 0) return;
  const int npc = max(0, (pos >> q.lgP) + 1 - q.n_local);
  if (npc <= p.K || p.K == 0) return;              // the selection kernel needs no keys for this row
  const int ntok = min(npc << q.lgP, pos + 1);
  const int t0 = blockIdx.x * kPkChunk;
  if (t0 >= ntok) return;
  const int t1 = min(t0 + kPkChunk, ntok);
  const int n = (t1 - t0 + (1 << q.lgP) - 1) >> q.lgP;
  const float* s = p.scores + b * p.ss[0] + g * p.ss[1] + r * p.ss[2];
  page_keys<kPkThreads>(s + t0, t1 - t0, q.lgP, n, pk);
  uint32_t* dst = pkg + (int64_t)row * npmax + (t0 >> q.lgP);
  for (int i = threadIdx.x; i < n; i += kPkThreads) dst[i] = pk[i];
}

// pkg: page keys from page_keys_kernel (row stride npmax), or null to
// compute them here.
__global__ __launch_bounds__(kPsThreads) void page_select_kernel(PageSelParams q, const uint32_t* pkg, int npmax) {
  constexpr int T = kPsThreads;
  __shared__ PsSmem sm;
  const TopkParams& p = q.t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x;
  const int r = row % p.Nq, g = (row / p.Nq) % p.G, b = row / (p.Nq * p.G);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  int32_t* out = p.idx + b * p.is[0] + g * p.is[1] + r * p.is[2];
  int32_t* cnt = p.count ? p.count + ((int64_t)b * p.G + g) * p.Nq + r : nullptr;
  const int W = q.width;
  if (pos < 0) {
    for (int i = tid; i < W; i += T) out[i] = -1;
    if (cnt && tid == 0) *cnt = 0;
    return;
  }
  const int lgP = q.lgP;
  const int last = pos >> lgP;
  const int npc = max(0, last + 1 - q.n_local);    // candidate pages 0..npc-1
  const int K = p.K;
  if (npc <= K) {                                   // every page is read
    for (int i = tid; i < W; i += T) out[i] = i <= last ? i : -1;
    if (cnt && tid == 0) *cnt = last + 1;
    return;
  }
  // from here npc > K, so the n_local recent pages all exist and W = K + n_local
  for (int i = tid; i < q.n_local; i += T) out[K + i] = npc + i;
  if (cnt && tid == 0) *cnt = K + q.n_local;
  if (K == 0) return;

  const float* s = p.scores + b * p.ss[0] + g * p.ss[1] + r * p.ss[2];
  if (pkg) {
    const uint32_t* src = pkg + (int64_t)row * npmax;
    for (int i = tid; i < npc; i += T) sm.pk[i] = src[i];
    __syncthreads();
  } else {
    page_keys<T>(s, min(npc << lgP, pos + 1), lgP, npc, sm.pk);
  }

  const uint32_t R = (uint32_t)K;
  uint32_t t, above;
  radix_select<T>(npc, R, [&](int i, uint32_t& k) { k = sm.pk[i]; return true; }, sm.hist, sm.sc, t, above);
  uint32_t klo = t, khi = t;
  float E = 0.f;
  IndexerRow ir{};
  if (p.certified) {
    const float tf = order_key_f32(t);
    ir = indexer_row(p.ix, b, g, r);
    // the row's bound: given, or (fused call) from the indexer's chunk maxima
    const float eps = p.err ? p.err[((int64_t)b * p.G + g) * p.Nq + r]
                            : row_eps(p.ix, ir, b, p.ix.G_k == 1 ? 0 : g, L, sm.red);
    E = 2.0f * eps * 1.0001f + 1e-30f;
    klo = f32_order_key(nextafterf(tf - E, -INFINITY));
    khi = f32_order_key(nextafterf(tf + E, INFINITY));
  }

  const int P = 1 << lgP;
  // lowest computed score a token may have and still hold the page's exact key
  auto tok_floor = [&](uint32_t ck) { return nextafterf(order_key_f32(ck) - E, -INFINITY); };

  // word pass: bits of the pages above the band (hist[w]) and in it (hist[512 + w]),
  // 64 pages per wave step
  static_assert(kMaxPages <= 32 * T && kMaxPages / 32 <= 512, "one bitmap word per thread");
  const int nwords = (npc + 31) >> 5;
  for (int c = (tid >> 6); 64 * c < npc; c += T / 64) {
    const int i = 64 * c + lane;
    const uint32_t k = i < npc ? sm.pk[i] : 0u;
    const uint64_t min_ = ballot(i < npc && k > khi);
    const uint64_t mbd = ballot(i < npc && k >= klo && k <= khi);
    if (lane == 0) {
      sm.hist[2 * c] = (uint32_t)min_;
      sm.hist[512 + 2 * c] = (uint32_t)mbd;
    } else if (lane == 1 && 2 * c + 1 < nwords) {
      sm.hist[2 * c + 1] = (uint32_t)(min_ >> 32);
      sm.hist[512 + 2 * c + 1] = (uint32_t)(mbd >> 32);
    }
  }
  __syncthreads();
  const uint32_t win = tid < nwords ? sm.hist[tid] : 0u;
  const uint32_t wbd = tid < nwords ? sm.hist[512 + tid] : 0u;
  uint32_t tot;
  const uint32_t pre = block_scan_sum<T>(((uint32_t)__popc(wbd) << 16) | (uint32_t)__popc(win), sm.sc, tot);
  const uint32_t n_in = tot & 0xFFFFu, n_band = tot >> 16;
  const uint32_t R2 = R - n_in;                    // >= 1: at most R-1 keys exceed t
  const bool cached = n_band <= (uint32_t)kPsBandCap;
  if (cached) {                                    // the band in page order
    uint32_t slot = pre >> 16;
    for (uint32_t m = wbd; m; m &= m - 1, ++slot) {
      const int i = 32 * tid + __ffs(m) - 1;
      sm.band_j[slot] = (uint32_t)i;
      sm.band_k[slot] = sm.pk[i];
    }
  }
  __syncthreads();

  // exact page key by one thread (the fallback beyond the band cache)
  auto exkey_thread = [&](int pg, uint32_t ck) -> uint32_t {
    if (!p.certified) return ck;
    const float lo = tok_floor(ck);
    const int j0 = pg << lgP, j1 = min(j0 + P, pos + 1);
    uint32_t bk = 0u;
    for (int j = j0; j < j1; ++j)
      if (s[j] >= lo) bk = max(bk, f32_order_key(exact_key(ir, j)));
    return bk;
  };

  if (!cached) {
    // rare (a band wider than the cache): exact keys recomputed by each thread
    // in an ordered pass over all pages
    uint32_t t2, above2;
    radix_select<T>(npc, R2,
                    [&](int i, uint32_t& k) {
                      const uint32_t ck = sm.pk[i];
                      if (ck < klo || ck > khi) return false;
                      k = exkey_thread(i, ck);
                      return true;
                    },
                    sm.hist, sm.sc, t2, above2);
    const uint32_t need_eq = R2 - above2;
    if (tid == 0) { sm.run[0] = 0; sm.run[2] = 0; }
    __syncthreads();
    for (int base = 0; base < npc; base += T) {
      const int i = base + tid;
      bool sel = false, eq = false;
      if (i < npc) {
        const uint32_t ck = sm.pk[i];
        sel = ck > khi;
        if (ck >= klo && ck <= khi) {
          const uint32_t ex = exkey_thread(i, ck);
          eq = ex == t2;
          sel = ex > t2;
        }
      }
      uint32_t neq;
      const uint32_t erank = sm.run[2] + block_prefix<T>(eq, sm.sc, neq);
      if (eq && erank < need_eq) sel = true;
      uint32_t nsel;
      const uint32_t opos = sm.run[0] + block_prefix<T>(sel, sm.sc, nsel);
      if (sel && opos < R) out[opos] = i;
      __syncthreads();
      if (tid == 0) { sm.run[0] += nsel; sm.run[2] += neq; }
      __syncthreads();
    }
    return;
  }

  if (p.certified) {
    // (band page, token) pairs whose token may hold the page's exact key,
    // listed in hist (tokens, then band slots); each pair is rescored by a
    // quarter-wave and folded into its page by an LDS maximum
    constexpr int kQCap = 2048;
    if (tid == 0) sm.run[2] = 0;
    __syncthreads();
    for (uint32_t e = tid >> 6; e < n_band; e += T / 64) {
      const float lo = tok_floor(sm.band_k[e]);
      const int j0 = (int)sm.band_j[e] << lgP, j1 = min(j0 + P, pos + 1);
      for (int jb = j0; jb < j1; jb += 64) {
        const int j = jb + lane;
        const uint64_t m = ballot(j < j1 && s[j] >= lo);
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&sm.run[2], (uint32_t)__popcll(m));
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        if ((m >> lane) & 1u) {
          const uint32_t slot = base + lanes_below(m);
          if (slot < (uint32_t)kQCap) {
            sm.hist[slot] = (uint32_t)j;
            sm.hist[kQCap + slot] = e;
          }
        }
      }
    }
    __syncthreads();
    const uint32_t nq = sm.run[2];
    if (nq <= (uint32_t)kQCap) {
      for (uint32_t e = tid; e < n_band; e += T) sm.band_k[e] = 0u;
      __syncthreads();
      for (uint32_t x = tid >> 4; x < nq; x += T / 16) {
        const float key = group_exact_key<16, 4, true>(ir, sm.hist[x]);
        if ((lane & 15) == 0) atomicMax(&sm.band_k[sm.hist[kQCap + x]], f32_order_key(key));
      }
    } else {                                       // many near-tied tokens: one wave per band page
      for (uint32_t e = tid >> 6; e < n_band; e += T / 64) {
        const float lo = tok_floor(sm.band_k[e]);
        const int j0 = (int)sm.band_j[e] << lgP, j1 = min(j0 + P, pos + 1);
        uint32_t bk = 0u;
        for (int jb = j0; jb < j1; jb += 64) {
          const int j = jb + lane;
          uint64_t m = ballot(j < j1 && s[j] >= lo);
          while (m) {
            const int bit = __builtin_ctzll(m);
            m &= m - 1;
            bk = max(bk, f32_order_key(wave_exact_key(ir, jb + bit)));
          }
        }
        if (lane == 0) sm.band_k[e] = bk;
      }
    }
    __syncthreads();
  }

  uint32_t t2, above2;
  radix_select<T>((int)n_band, R2, [&](int i, uint32_t& k) { k = sm.band_k[i]; return true; }, sm.hist, sm.sc,
                  t2, above2);
  const uint32_t need_eq = R2 - above2;

  // selection bitmap (in pk, whose keys are no longer needed): the pages above
  // the band, then the band's winners in page order
  sm.pk[tid] = win;
  __syncthreads();
  uint32_t run_eq = 0;
  for (uint32_t base = 0; base < n_band; base += T) {
    const uint32_t e = base + tid;
    const uint32_t ex = e < n_band ? sm.band_k[e] : 0u;
    const bool eq = e < n_band && ex == t2;
    uint32_t neq;
    const uint32_t er = run_eq + block_prefix<T>(eq, sm.sc, neq);
    run_eq += neq;
    if (e < n_band && (ex > t2 || (eq && er < need_eq))) {
      const uint32_t i = sm.band_j[e];
      atomicOr(&sm.pk[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
  const uint32_t wsel = tid < nwords ? sm.pk[tid] : 0u;
  uint32_t nsel;
  uint32_t opos = block_scan_sum<T>((uint32_t)__popc(wsel), sm.sc, nsel);
  for (uint32_t m = wsel; m; m &= m - 1, ++opos)
    if (opos < R) out[opos] = 32 * tid + __ffs(m) - 1;
}

static int page_rows(const PageSelParams& p) { return p.t.B * p.t.G * p.t.Nq; }
static int page_cap(const PageSelParams& p) { return (p.t.ctx + (1 << p.lgP) - 1) >> p.lgP; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout. Fused: scores [B, G, Nq, ctx] f32 | the indexer's chunk
// maxima of |k| | page keys [rows][pages]. Otherwise the page
// keys only, and only for few rows.
struct PsLayout {
  size_t scores, kmax, keys, total;
  bool staged;             // page keys staged in the workspace
  bool epilogue;           // ... by the indexer itself
};

static PsLayout ps_layout(const PageSelParams& p) {
  PsLayout l{};
  const size_t rows = (size_t)page_rows(p);
  size_t off = 0;
  if (p.fused) {
    l.scores = off;
    off += align256(rows * p.t.ctx * sizeof(float));
    l.kmax = off;
    off += align256(indexer_ws_bytes(p.t.ix.B, p.t.ix.G_k, p.t.ix.ctx));
    l.epilogue = index_pagekeys_ok(p.t.ix, p.lgP);
  }
  l.staged = l.epilogue || rows <= (size_t)kPsFewRows;
  l.keys = off;
  if (l.staged) off += rows * page_cap(p) * sizeof(uint32_t);
  l.total = off;
  return l;
}

size_t page_select_ws_bytes(const PageSelParams& p) { return ps_layout(p).total; }

hipError_t launch_page_select(const PageSelParams& p0, hipStream_t st) {
  PageSelParams p = p0;
  const int rows = page_rows(p);
  const int npmax = page_cap(p);
  const PsLayout l = ps_layout(p);
  char* w = (char*)p.ws;
  uint32_t* pkg = l.staged ? (uint32_t*)(w + l.keys) : nullptr;
  hipError_t e;
  if (p.fused) {
    IndexerParams x = p.t.ix;
    x.scores = (float*)(w + l.scores);
    x.ss[3] = 1;
    x.ss[2] = p.t.ctx;
    x.ss[1] = (int64_t)p.t.Nq * p.t.ctx;
    x.ss[0] = (int64_t)p.t.G * p.t.Nq * p.t.ctx;
    x.err = nullptr;                  // the selection kernel bounds each row itself
    x.kmax = (float*)(w + l.kmax);
    x.chunk = index_chunk(x);
    x.nchunk = (x.ctx + x.chunk - 1) / x.chunk;
    if (l.epilogue) {
      x.pkeys = pkg;
      x.pk_stride = npmax;
      x.pk_lgP = p.lgP;
    }
    if ((e = launch_index_scores(x, st)) != hipSuccess) return e;
    p.t.scores = x.scores;
    for (int i = 0; i < 4; ++i) p.t.ss[i] = x.ss[i];
    p.t.err = nullptr;
    p.t.certified = true;
    p.t.ix = x;
  }
  if (pkg && !l.epilogue) {
    const int chunks = (p.t.ctx + kPkChunk - 1) / kPkChunk;
    hipLaunchKernelGGL(page_keys_kernel, dim3(chunks, rows), dim3(kPkThreads), 0, st, p, pkg, npmax);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(page_select_kernel, dim3(rows), dim3(kPsThreads), 0, st, p, (const uint32_t*)pkg, npmax);
  return hipGetLastError();
}

hipError_t launch_page_select_keys(const PageSelParams& p, const uint32_t* pkg, int npmax, hipStream_t st) {
  hipLaunchKernelGGL(page_select_kernel, dim3(page_rows(p)), dim3(kPsThreads), 0, st, p, pkg, npmax);
  return hipGetLastError();
}

}  // namespace sp
