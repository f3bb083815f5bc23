// Per-row top-K with lower-index tie breaking, optionally certified.
//
// Row (b, g, r) has candidates 0..p. With t the K-th largest score:
//  * uncertified: selected = {s > t} plus the lowest-index elements with s == t;
//  * certified (scores s~ carry a bound |s~ - key| <= eps, key = float32
//    nearest to the exact score): every element with s~ > t + 2 eps is in the
//    exact top-K and none with s~ < t - 2 eps is; the band in between is
//    rescored exactly and the remaining slots go to the band's best by
//    (exact key desc, index asc).
// Output indices are ascending, -1 padded.
//
// Two schedules:
//  * many rows: one 512-thread workgroup per row (radix select in LDS over the
//    row, ordered compaction), the band cached in LDS or recomputed.
//  * few long rows (decode): C workgroups per row.
//      mt_hist:     12-bit histogram of the row into global memory; the last
//                   workgroup of a row to finish finds the bin holding the K-th
//                   largest key.
//      mt_collect:  elements above that bin (plus the certification margin)
//                   become bits of a per-row bitmap; elements in it become a
//                   short candidate list.
//      mt_finalize: one workgroup per row resolves the candidates (exactly,
//                   when certified), sets their bits, and writes the bitmap out
//                   as ascending indices.
#include "common.h"
#include "exact.h"
#include "internal.h"
#include "rowselect.h"

namespace sp {

constexpr int kTkThreads = 512;
constexpr int kBandCap = 2048;
constexpr int kMtChunk = 8192;      // elements per workgroup in the multi-workgroup schedule
constexpr int kMtThreads = 256;
constexpr int kCandCap = 4096;      // candidates per row cached by mt_finalize

struct RowSmem {
  uint32_t hist[4096];
  uint32_t band_j[kBandCap];
  uint32_t band_k[kBandCap];
  uint32_t sc[16];
  uint32_t run[4];
};

struct RowCtx {
  int b, g, r, n;
  const float* s;
  int32_t* out;
  uint32_t klo, khi;     // band limits as order keys (set after t is known)
  IndexerRow ir;
};

SP_DEV RowCtx row_ctx(const TopkParams& p, int row) {
  RowCtx c;
  c.r = row % p.Nq;
  c.g = (row / p.Nq) % p.G;
  c.b = row / (p.Nq * p.G);
  const int L = min(p.ctx_len ? p.ctx_len[c.b] : p.ctx, p.ctx);
  c.n = min(L - p.Nq + c.r + 1, p.ctx);
  c.out = p.idx + c.b * p.is[0] + c.g * p.is[1] + c.r * p.is[2];
  c.s = p.scores + c.b * p.ss[0] + c.g * p.ss[1] + c.r * p.ss[2];
  c.ir = IndexerRow{};
  if (p.certified) {
    const IndexerParams& x = p.ix;
    const int hpg = x.hpg;
    const int kg = x.G_k == 1 ? 0 : c.g;
    const int esz = x.q.dt == DT_F32 ? 4 : 2;
    const int ksz = x.k.dt == DT_F32 ? 4 : (x.k.dt == DT_BF16 ? 2 : 1);
    c.ir.q = (const char*)x.q.p + (c.b * x.q.s[0] + c.r * x.q.s[1] + (int64_t)c.g * hpg * x.q.s[2]) * esz;
    c.ir.qt = x.q.dt;
    c.ir.qh_stride = x.q.s[2];
    c.ir.k = (const char*)x.k.p + (c.b * x.k.s[0] + kg * x.k.s[2]) * ksz;
    c.ir.kt = x.k.dt;
    c.ir.k_stride = x.k.s[1];
    c.ir.w = x.relu ? x.w + c.b * x.ws_[0] + c.r * x.ws_[1] + (int64_t)c.g * hpg * x.ws_[2] : nullptr;
    c.ir.w_stride = x.ws_[2];
    c.ir.H = hpg;
    c.ir.d = x.d_I;
    c.ir.relu = x.relu;
  }
  return c;
}

// order-key limits of the band [t - 2 eps, t + 2 eps], rounded outward
SP_DEV void band_limits(const TopkParams& p, const RowCtx& c, float tf, float lo_f, float hi_f,
                        uint32_t& klo, uint32_t& khi) {
  if (!p.certified) {
    klo = f32_order_key(lo_f);
    khi = f32_order_key(hi_f);
    return;
  }
  const float eps = p.err[((int64_t)c.b * p.G + c.g) * p.Nq + c.r];
  const float E = 2.0f * eps * 1.0001f + 1e-30f;
  klo = f32_order_key(nextafterf(lo_f - E, -INFINITY));
  khi = f32_order_key(nextafterf(hi_f + E, INFINITY));
  (void)tf;
}

SP_DEV uint32_t exkey_of(const TopkParams& p, const RowCtx& c, int j, uint32_t ks) {
  return p.certified ? f32_order_key(exact_key(c.ir, j)) : ks;
}

// The whole selection for one row by one workgroup of T threads.
template <int T>
SP_DEV void row_topk_single(const TopkParams& p, RowCtx& c, RowSmem& sm) {
  const int tid = threadIdx.x;
  const int n = c.n, K = p.K;
  const float* s = c.s;
  auto skey = [&](int i) -> uint32_t { return f32_order_key(s[i]); };
  uint32_t t, above;
  radix_select<T>(n, (uint32_t)K, [&](int i, uint32_t& k) { k = skey(i); return true; }, sm.hist, sm.sc, t,
                  above);
  const float tf = order_key_f32(t);
  uint32_t klo, khi;
  band_limits(p, c, tf, tf, tf, klo, khi);

  // ordered pass 1: count elements above the band, cache the band
  if (tid == 0) { sm.run[0] = 0; sm.run[1] = 0; }
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
    const uint32_t bpos = block_prefix<T>(bd, sm.sc, nbd);
    block_prefix<T>(in, sm.sc, nin);
    const uint32_t bslot = sm.run[1] + bpos;
    if (bd && bslot < kBandCap) {
      sm.band_j[bslot] = j;
      sm.band_k[bslot] = exkey_of(p, c, j, ks);
    }
    __syncthreads();
    if (tid == 0) { sm.run[0] += nin; sm.run[1] += nbd; }
    __syncthreads();
  }
  const uint32_t n_in = sm.run[0], n_band = sm.run[1];
  const uint32_t R = (uint32_t)K - n_in;   // >= 1
  const bool cached = n_band <= (uint32_t)kBandCap;

  uint32_t t2, above2;
  if (cached) {
    radix_select<T>((int)n_band, R, [&](int i, uint32_t& k) { k = sm.band_k[i]; return true; }, sm.hist, sm.sc,
                    t2, above2);
  } else {
    radix_select<T>(n, R,
                    [&](int i, uint32_t& k) {
                      const uint32_t ks = skey(i);
                      if (ks < klo || ks > khi) return false;
                      k = exkey_of(p, c, i, ks);
                      return true;
                    },
                    sm.hist, sm.sc, t2, above2);
  }
  const uint32_t need_eq = R - above2;

  // ordered pass 2: write the selection in ascending index order
  if (tid == 0) { sm.run[0] = 0; sm.run[1] = 0; sm.run[2] = 0; }
  __syncthreads();
  for (int base = 0; base < n; base += T) {
    const int j = base + tid;
    bool sel = false, bd = false, eq = false;
    if (j < n) {
      const uint32_t ks = skey(j);
      sel = ks > khi;
      bd = ks >= klo && ks <= khi;
    }
    uint32_t nbd;
    const uint32_t brank = sm.run[1] + block_prefix<T>(bd, sm.sc, nbd);
    if (bd) {
      const uint32_t ex = cached ? sm.band_k[brank] : exkey_of(p, c, j, skey(j));
      eq = ex == t2;
      if (ex > t2) sel = true;
    }
    uint32_t neq;
    const uint32_t erank = sm.run[2] + block_prefix<T>(eq, sm.sc, neq);
    if (eq && erank < need_eq) sel = true;
    uint32_t nsel;
    const uint32_t opos = sm.run[0] + block_prefix<T>(sel, sm.sc, nsel);
    if (sel && opos < (uint32_t)K) c.out[opos] = j;
    __syncthreads();
    if (tid == 0) { sm.run[0] += nsel; sm.run[1] += nbd; sm.run[2] += neq; }
    __syncthreads();
  }
}

SP_DEV void write_all(const TopkParams& p, const RowCtx& c, int T) {
  for (int i = threadIdx.x; i < p.K; i += T) c.out[i] = i < c.n ? i : -1;
  if (p.count && threadIdx.x == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = max(c.n, 0);
}

__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(TopkParams p) {
  __shared__ RowSmem sm;
  RowCtx c = row_ctx(p, blockIdx.x);
  if (c.n <= p.K) return write_all(p, c, kTkThreads);
  row_topk_single<kTkThreads>(p, c, sm);
  if (p.count && threadIdx.x == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
}

// ---------------------------------------------------------------- multi-workgroup schedule
struct MtWs {
  uint32_t* hist;     // [rows][4096]
  uint32_t* ctr;      // [rows][8]: done, n_above, n_cand, bin, above_bin
  uint32_t* bitmap;   // [rows][words]
  uint32_t* cand_k;   // [rows][kCandCap]
  uint32_t* cand_j;   // [rows][kCandCap]
  int words, nchunk;
};

SP_DEV uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void mt_zero_kernel(MtWs w) {
  uint32_t* h = w.hist + (int64_t)blockIdx.x * 4096;
  for (int i = threadIdx.x; i < 4096; i += 256) h[i] = 0;
  if (threadIdx.x < 8) w.ctr[blockIdx.x * 8 + threadIdx.x] = 0;
}

__global__ __launch_bounds__(kMtThreads) void mt_hist_kernel(TopkParams p, MtWs w) {
  __shared__ uint32_t h[4096];
  __shared__ uint32_t sc[16];
  __shared__ int last;
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  RowCtx c = row_ctx(p, row);
  if (c.n <= p.K) return;   // whole row handled by mt_finalize
  for (int i = tid; i < 4096; i += kMtThreads) h[i] = 0;
  __syncthreads();
  const int j0 = chunk * kMtChunk, j1 = min(c.n, j0 + kMtChunk);
  for (int j = j0 + tid; j < j1; j += kMtThreads) atomicAdd(&h[f32_order_key(c.s[j]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = w.hist + (int64_t)row * 4096;
  for (int i = tid; i < 4096; i += kMtThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(&w.ctr[row * 8 + 0], 1u) == (uint32_t)(w.nchunk - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  // the last workgroup: find the bin holding the K-th largest key
  for (int i = tid; i < 4096; i += kMtThreads) h[i] = ld_agent(&gh[i]);
  __syncthreads();
  constexpr int per = 4096 / kMtThreads;
  const int lo = tid * per;
  uint32_t mine = 0;
  for (int q = 0; q < per; ++q) mine += h[lo + q];
  uint32_t tot;
  // suffix sums: reverse the thread order through the prefix helper
  const uint32_t excl_rev = block_scan_sum<kMtThreads>(mine, sc, tot);   // sum over lower threads
  uint32_t cum = tot - excl_rev - mine;                                   // sum over higher bins
  const uint32_t K = (uint32_t)p.K;
  if (cum < K && cum + mine >= K) {
    for (int q = per - 1; q >= 0; --q) {
      const uint32_t hv = h[lo + q];
      if (cum + hv >= K) {
        w.ctr[row * 8 + 3] = (uint32_t)(lo + q);
        w.ctr[row * 8 + 4] = cum;
        break;
      }
      cum += hv;
    }
  }
}

__global__ __launch_bounds__(kMtThreads) void mt_collect_kernel(TopkParams p, MtWs w) {
  __shared__ uint32_t bm[kMtChunk / 32];
  __shared__ uint32_t sc[16];
  __shared__ uint32_t cbase;
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  RowCtx c = row_ctx(p, row);
  if (c.n <= p.K) return;
  const int j0 = chunk * kMtChunk;
  if (j0 >= c.n) return;
  const int j1 = min(c.n, j0 + kMtChunk);
  const uint32_t bin = w.ctr[row * 8 + 3];
  const float lo_b = order_key_f32(bin << 20), hi_b = order_key_f32((bin << 20) | 0xFFFFFu);
  uint32_t klo, khi;
  band_limits(p, c, 0.f, lo_b, hi_b, klo, khi);
  for (int i = tid; i < kMtChunk / 32; i += kMtThreads) bm[i] = 0;
  __syncthreads();
  uint32_t n_above = 0;
  for (int base = j0; base < j1; base += kMtThreads) {
    const int j = base + tid;
    bool cand = false;
    uint32_t ks = 0;
    if (j < j1) {
      ks = f32_order_key(c.s[j]);
      if (ks > khi) {
        atomicOr(&bm[(j - j0) >> 5], 1u << (j & 31));
        ++n_above;
      }
      cand = ks >= klo && ks <= khi;
    }
    uint32_t ncand;
    const uint32_t pos = block_prefix<kMtThreads>(cand, sc, ncand);
    if (ncand) {
      if (tid == 0) cbase = atomicAdd(&w.ctr[row * 8 + 2], ncand);
      __syncthreads();
      const uint32_t slot = cbase + pos;
      if (cand && slot < (uint32_t)kCandCap) {
        w.cand_k[(int64_t)row * kCandCap + slot] = ks;
        w.cand_j[(int64_t)row * kCandCap + slot] = j;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  uint32_t tot;
  block_scan_sum<kMtThreads>(n_above, sc, tot);
  if (tid == 0 && tot) atomicAdd(&w.ctr[row * 8 + 1], tot);
  uint32_t* gb = w.bitmap + (int64_t)row * w.words + (j0 >> 5);
  const int nw = (j1 - j0 + 31) >> 5;
  for (int i = tid; i < nw; i += kMtThreads) gb[i] = bm[i];
}

struct FinSmem {
  RowSmem row;
  uint32_t ck[kCandCap];
  uint32_t cj[kCandCap];
};

__global__ __launch_bounds__(kTkThreads) void mt_finalize_kernel(TopkParams p, MtWs w) {
  constexpr int T = kTkThreads;
  __shared__ FinSmem sm;
  const int row = blockIdx.x, tid = threadIdx.x;
  RowCtx c = row_ctx(p, row);
  if (c.n <= p.K) return write_all(p, c, T);
  const uint32_t n_above = w.ctr[row * 8 + 1];
  const uint32_t n_cand = w.ctr[row * 8 + 2];
  if (n_cand > (uint32_t)kCandCap) {          // too many near the threshold: do the row in one pass
    row_topk_single<T>(p, c, sm.row);
    if (p.count && tid == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
    return;
  }
  for (uint32_t i = tid; i < n_cand; i += T) {
    sm.ck[i] = w.cand_k[(int64_t)row * kCandCap + i];
    sm.cj[i] = w.cand_j[(int64_t)row * kCandCap + i];
  }
  __syncthreads();
  const uint32_t R = (uint32_t)p.K - n_above;
  uint32_t t, above;
  radix_select<T>((int)n_cand, R, [&](int i, uint32_t& k) { k = sm.ck[i]; return true; }, sm.row.hist,
                  sm.row.sc, t, above);
  const float tf = order_key_f32(t);
  uint32_t klo, khi;
  band_limits(p, c, tf, tf, tf, klo, khi);
  // candidates above the band are in; band members get exact keys
  uint32_t* gb = w.bitmap + (int64_t)row * w.words;
  uint32_t n_in = 0;
  for (uint32_t i = tid; i < n_cand; i += T) {
    const uint32_t ks = sm.ck[i];
    if (ks > khi) {
      atomicOr(&gb[sm.cj[i] >> 5], 1u << (sm.cj[i] & 31));
      ++n_in;
      sm.ck[i] = 0;                     // marks "decided"
    } else if (ks >= klo) {
      sm.ck[i] = exkey_of(p, c, (int)sm.cj[i], ks) | 0u;
      sm.cj[i] |= 0x80000000u;          // band member
    } else {
      sm.ck[i] = 0;
    }
  }
  uint32_t tot_in;
  block_scan_sum<T>(n_in, sm.row.sc, tot_in);
  const uint32_t R2 = R - tot_in;
  // best R2 band members by (exact key desc, index asc)
  uint32_t t2, above2;
  radix_select<T>((int)n_cand,
                  R2, [&](int i, uint32_t& k) { k = sm.ck[i]; return (sm.cj[i] & 0x80000000u) != 0; },
                  sm.row.hist, sm.row.sc, t2, above2);
  const uint32_t need_eq = R2 - above2;
  for (uint32_t i = tid; i < n_cand; i += T) {
    if (!(sm.cj[i] & 0x80000000u)) continue;
    const uint32_t j = sm.cj[i] & 0x7FFFFFFFu, k = sm.ck[i];
    bool sel = k > t2;
    if (k == t2) {
      uint32_t rank = 0;   // equal exact keys with a lower index
      for (uint32_t f = 0; f < n_cand; ++f)
        rank += ((sm.cj[f] & 0x80000000u) && sm.ck[f] == t2 && (sm.cj[f] & 0x7FFFFFFFu) < j) ? 1u : 0u;
      sel = rank < need_eq;
    }
    if (sel) atomicOr(&gb[j >> 5], 1u << (j & 31));
  }
  __threadfence();
  __syncthreads();
  // bitmap -> ascending indices
  const int nwords = (c.n + 31) >> 5;
  const int per = (nwords + T - 1) / T;
  const int w0 = tid * per, w1 = min(nwords, w0 + per);
  uint32_t cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(ld_agent(&gb[i]));
  uint32_t total;
  uint32_t pos = block_scan_sum<T>(cnt, sm.row.sc, total);
  for (int i = w0; i < w1; ++i) {
    uint32_t m = ld_agent(&gb[i]);
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (pos < (uint32_t)p.K) c.out[pos] = i * 32 + bit;
      ++pos;
    }
  }
  for (int i = (int)total + tid; i < p.K; i += T) c.out[i] = -1;
  if (p.count && tid == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = (int)min(total, (uint32_t)p.K);
}

static bool use_multi(const TopkParams& p) {
  const int64_t rows = (int64_t)p.B * p.G * p.Nq;
  return rows <= 1024 && p.ctx >= 4 * kMtChunk;
}

size_t topk_ws_bytes(const TopkParams& p) {
  if (!use_multi(p)) return 0;
  const int64_t rows = (int64_t)p.B * p.G * p.Nq;
  const int64_t words = (p.ctx + 31) / 32;
  return (size_t)rows * (4096 + 8 + words + 2 * kCandCap) * sizeof(uint32_t);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const int rows = p.B * p.G * p.Nq;
  if (!use_multi(p)) {
    hipLaunchKernelGGL(topk_row_kernel, dim3(rows), dim3(kTkThreads), 0, st, p);
    return hipGetLastError();
  }
  MtWs w;
  w.words = (p.ctx + 31) / 32;
  w.nchunk = (p.ctx + kMtChunk - 1) / kMtChunk;
  uint32_t* base = (uint32_t*)p.ws;
  w.hist = base;
  w.ctr = w.hist + (int64_t)rows * 4096;
  w.bitmap = w.ctr + (int64_t)rows * 8;
  w.cand_k = w.bitmap + (int64_t)rows * w.words;
  w.cand_j = w.cand_k + (int64_t)rows * kCandCap;
  hipLaunchKernelGGL(mt_zero_kernel, dim3(rows), dim3(256), 0, st, w);
  hipLaunchKernelGGL(mt_hist_kernel, dim3(w.nchunk, rows), dim3(kMtThreads), 0, st, p, w);
  hipLaunchKernelGGL(mt_collect_kernel, dim3(w.nchunk, rows), dim3(kMtThreads), 0, st, p, w);
  hipLaunchKernelGGL(mt_finalize_kernel, dim3(rows), dim3(kTkThreads), 0, st, p, w);
  return hipGetLastError();
}

}  // namespace sp
