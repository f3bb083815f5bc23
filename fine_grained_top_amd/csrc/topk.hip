// Per-row top-K with lower-index tie breaking, optionally certified.
//
// One workgroup (512 threads) per (request, group, query row). The row's
// candidates are keys 0..p. Radix select finds t, the K-th largest score.
//
// Uncertified: selected = {s > t} plus the lowest-index elements with s == t.
//
// Certified (scores s~ carry a bound |s~ - key| <= eps, key = float32 nearest
// to the exact score): every element with s~ > t + 2 eps is in the exact
// top-K, none with s~ < t - 2 eps is; the band in between is rescored exactly
// and the remaining K - |in| slots go to the band's best by
// (exact key desc, index asc). The band is cached in LDS when it fits and
// recomputed on the fly otherwise, so any band size is handled exactly.
// The output is written in ascending index order by ordered compaction.
#include "common.h"
#include "exact.h"
#include "internal.h"
#include "rowselect.h"

namespace sp {

constexpr int kTkThreads = 512;
constexpr int kBandCap = 2048;

__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(TopkParams p) {
  constexpr int T = kTkThreads;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t band_j[kBandCap];
  __shared__ uint32_t band_k[kBandCap];
  __shared__ uint32_t sc[16];
  __shared__ uint32_t run[4];

  const int row = blockIdx.x;
  const int r = row % p.Nq;
  const int g = (row / p.Nq) % p.G;
  const int b = row / (p.Nq * p.G);
  const int tid = threadIdx.x;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int n = min(L - p.Nq + r + 1, p.ctx);     // candidates 0..p
  int32_t* out = p.idx + b * p.is[0] + g * p.is[1] + r * p.is[2];
  const float* s = p.scores + b * p.ss[0] + g * p.ss[1] + r * p.ss[2];
  const int K = p.K;

  if (n <= K) {   // everything is selected
    for (int i = tid; i < K; i += T) out[i] = i < n ? i : -1;
    if (p.count && tid == 0) p.count[(b * p.G + g) * p.Nq + r] = max(n, 0);
    return;
  }

  auto skey = [&](int i) -> uint32_t { return f32_order_key(s[i]); };
  uint32_t t, above;
  radix_select<T>(n, (uint32_t)K, [&](int i, uint32_t& k) { k = skey(i); return true; }, hist, sc, t,
                  above);

  // band limits
  uint32_t klo = t, khi = t;
  IndexerRow ir{};
  if (p.certified) {
    const float eps = p.err[(b * p.G + g) * p.Nq + r];
    const float tf = order_key_f32(t);
    const float E = 2.0f * eps * 1.0001f + 1e-30f;
    const float lo = nextafterf(tf - E, -INFINITY);
    const float hi = nextafterf(tf + E, INFINITY);
    klo = f32_order_key(lo);
    khi = f32_order_key(hi);
    const IndexerParams& x = p.ix;
    const int hpg = x.hpg;
    const int kg = x.G_k == 1 ? 0 : g;
    const int esz = x.q.dt == DT_F32 ? 4 : 2;
    const int ksz = x.k.dt == DT_F32 ? 4 : (x.k.dt == DT_BF16 ? 2 : 1);
    ir.q = (const char*)x.q.p + (b * x.q.s[0] + r * x.q.s[1] + (int64_t)g * hpg * x.q.s[2]) * esz;
    ir.qt = x.q.dt;
    ir.qh_stride = x.q.s[2];
    ir.k = (const char*)x.k.p + (b * x.k.s[0] + kg * x.k.s[2]) * ksz;
    ir.kt = x.k.dt;
    ir.k_stride = x.k.s[1];
    ir.w = x.relu ? x.w + b * x.ws_[0] + r * x.ws_[1] + (int64_t)g * hpg * x.ws_[2] : nullptr;
    ir.w_stride = x.ws_[2];
    ir.H = hpg;
    ir.d = x.d_I;
    ir.relu = x.relu;
  }
  auto exkey = [&](int j, uint32_t ks) -> uint32_t {
    return p.certified ? f32_order_key(exact_key(ir, j)) : ks;
  };

  // ordered pass 1: count elements above the band, cache the band
  if (tid == 0) { run[0] = 0; run[1] = 0; }
  __syncthreads();
  for (int base = 0; base < n; base += T) {
    const int j = base + tid;
    uint32_t ks = 0;
    bool in = false, bd = false;
    if (j < n) {
      ks = skey(j);
      in = ks > khi;
      bd = ks >= klo && ks <= khi;
    }
    uint32_t nin, nbd;
    const uint32_t bpos = block_prefix<T>(bd, sc, nbd);
    block_prefix<T>(in, sc, nin);
    const uint32_t bslot = run[1] + bpos;
    if (bd && bslot < kBandCap) {
      band_j[bslot] = j;
      band_k[bslot] = exkey(j, ks);
    }
    __syncthreads();
    if (tid == 0) { run[0] += nin; run[1] += nbd; }
    __syncthreads();
  }
  const uint32_t n_in = run[0], n_band = run[1];
  const uint32_t R = (uint32_t)K - n_in;   // >= 1
  const bool cached = n_band <= (uint32_t)kBandCap;

  uint32_t t2, above2;
  if (cached) {
    radix_select<T>((int)n_band, R, [&](int i, uint32_t& k) { k = band_k[i]; return true; }, hist, sc,
                    t2, above2);
  } else {
    radix_select<T>(n, R,
                    [&](int i, uint32_t& k) {
                      const uint32_t ks = skey(i);
                      if (ks < klo || ks > khi) return false;
                      k = exkey(i, ks);
                      return true;
                    },
                    hist, sc, t2, above2);
  }
  const uint32_t need_eq = R - above2;

  // ordered pass 2: write the selection in ascending index order
  if (tid == 0) { run[0] = 0; run[1] = 0; run[2] = 0; }
  __syncthreads();
  for (int base = 0; base < n; base += T) {
    const int j = base + tid;
    bool sel = false, bd = false, eq = false;
    uint32_t ex = 0;
    if (j < n) {
      const uint32_t ks = skey(j);
      sel = ks > khi;
      bd = ks >= klo && ks <= khi;
    }
    uint32_t nbd;
    const uint32_t brank = run[1] + block_prefix<T>(bd, sc, nbd);
    if (bd) {
      ex = cached ? band_k[brank] : exkey(j, skey(j));
      eq = ex == t2;
      if (ex > t2) sel = true;
    }
    uint32_t neq;
    const uint32_t erank = run[2] + block_prefix<T>(eq, sc, neq);
    if (eq && erank < need_eq) sel = true;
    uint32_t nsel;
    const uint32_t opos = run[0] + block_prefix<T>(sel, sc, nsel);
    if (sel && opos < (uint32_t)K) out[opos] = j;
    __syncthreads();
    if (tid == 0) { run[0] += nsel; run[1] += nbd; run[2] += neq; }
    __syncthreads();
  }
  if (p.count && tid == 0) p.count[(b * p.G + g) * p.Nq + r] = K;
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const int rows = p.B * p.G * p.Nq;
  hipLaunchKernelGGL(topk_row_kernel, dim3(rows), dim3(kTkThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sp
