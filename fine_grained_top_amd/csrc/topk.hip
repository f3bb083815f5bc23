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
//      mt_hist:     12-bit histogram of the row, added into global memory.
//      mt_collect:  every workgroup finds the bin holding the K-th largest key
//                   from that histogram; elements above the bin (plus the
//                   certification margin) become bits of a per-row bitmap,
//                   elements in it a short candidate list.
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
constexpr int kCandCap = 8192;      // candidates per row cached by mt_finalize

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
      sm.band_k[bslot] = ks;
    }
    __syncthreads();
    if (tid == 0) { sm.run[0] += nin; sm.run[1] += nbd; }
    __syncthreads();
  }
  const uint32_t n_in = sm.run[0], n_band = sm.run[1];
  const uint32_t R = (uint32_t)K - n_in;   // >= 1
  const bool cached = n_band <= (uint32_t)kBandCap;
  if (cached && p.certified) {            // exact keys of the band, one wave per member
    for (uint32_t e = tid >> 6; e < n_band; e += T / 64) {
      const float key = wave_exact_key(c.ir, sm.band_j[e]);
      if ((tid & 63) == 0) sm.band_k[e] = f32_order_key(key);
    }
    __syncthreads();
  }

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
// Workgroups of one row communicate only across kernel boundaries (no
// device-scope fences or returning atomics inside a kernel): histogram
// atomics land in global memory and the next kernel reads them; every chunk
// owns fixed slots for its counts and candidates.
constexpr int kMaxWords = 8192;     // bitmap words per row cached in LDS (rows up to 262144 keys)
constexpr int kChunkCand = 512;     // candidate slots per chunk

struct MtWs {
  uint32_t* hist;     // [rows][4096]
  uint32_t* cnt;      // [rows][nchunk][2]: keys above the window, candidates
  uint32_t* bin;      // [rows]
  uint32_t* bitmap;   // [rows][words]
  uint32_t* cand_k;   // [rows][nchunk][kChunkCand]
  uint32_t* cand_j;   // [rows][nchunk][kChunkCand]
  int words, nchunk;
};

__global__ __launch_bounds__(256) void mt_zero_kernel(MtWs w) {
  uint32_t* h = w.hist + (int64_t)blockIdx.x * 4096;
  for (int i = threadIdx.x; i < 4096; i += 256) h[i] = 0;
}

__global__ __launch_bounds__(kMtThreads) void mt_hist_kernel(TopkParams p, MtWs w) {
  __shared__ uint32_t h[4096];
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  RowCtx c = row_ctx(p, row);
  const int j0 = chunk * kMtChunk, j1 = min(c.n, j0 + kMtChunk);
  if (c.n <= p.K || j0 >= j1) return;
  for (int i = tid; i < 4096; i += kMtThreads) h[i] = 0;
  __syncthreads();
  for (int j = j0 + tid; j < j1; j += kMtThreads) atomicAdd(&h[f32_order_key(c.s[j]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = w.hist + (int64_t)row * 4096;
  for (int i = tid; i < 4096; i += kMtThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// window of order keys holding every candidate: the threshold bin, widened
// by the certification margin
SP_DEV void cand_window(const TopkParams& p, const RowCtx& c, uint32_t bin, uint32_t& klo, uint32_t& khi) {
  const float lo_b = order_key_f32(bin << 20), hi_b = order_key_f32((bin << 20) | 0xFFFFFu);
  band_limits(p, c, 0.f, lo_b, hi_b, klo, khi);
}

__global__ __launch_bounds__(kMtThreads) void mt_collect_kernel(TopkParams p, MtWs w) {
  __shared__ uint32_t sc[16];
  __shared__ uint32_t binsel;
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  RowCtx c = row_ctx(p, row);
  const int j0 = chunk * kMtChunk;
  if (c.n <= p.K || j0 >= c.n) return;
  const int j1 = min(c.n, j0 + kMtChunk);
  constexpr int PER = kMtChunk / kMtThreads;   // elements per thread, kept in registers
  uint32_t ks[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = j0 + i * kMtThreads + tid;
    ks[i] = j < j1 ? f32_order_key(c.s[j]) : 0u;
  }
  // bin holding the K-th largest key, from the row histogram
  {
    const uint32_t* gh = w.hist + (int64_t)row * 4096;
    constexpr int per = 4096 / kMtThreads;
    const int lo = tid * per;
    uint32_t hv[per], mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
      hv[q] = gh[lo + q];
      mine += hv[q];
    }
    uint32_t tot;
    const uint32_t below = block_scan_sum<kMtThreads>(mine, sc, tot);
    uint32_t cum = tot - below - mine;              // keys in higher bins
    const uint32_t K = (uint32_t)p.K;
    if (cum < K && cum + mine >= K) {
      for (int q = per - 1; q >= 0; --q) {
        if (cum + hv[q] >= K) {
          binsel = (uint32_t)(lo + q);
          break;
        }
        cum += hv[q];
      }
    }
  }
  __syncthreads();
  const uint32_t bin = binsel;
  if (chunk == 0 && tid == 0) w.bin[row] = bin;
  uint32_t klo, khi;
  cand_window(p, c, bin, klo, khi);
  // bitmap words straight from ballots: a wave's 64 consecutive elements are 2 words
  uint32_t* gb = w.bitmap + (int64_t)row * w.words;
  uint32_t ncand = 0, n_above = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = j0 + i * kMtThreads + tid;
    const bool above = j < j1 && ks[i] > khi;
    ncand += (j < j1 && ks[i] >= klo && ks[i] <= khi) ? 1u : 0u;
    const uint64_t m = ballot(above);
    const int jw = j0 + i * kMtThreads + (tid & ~63);
    if (lane == 0 && jw < j1) gb[jw >> 5] = (uint32_t)m;
    if (lane == 32 && jw + 32 < j1) gb[(jw >> 5) + 1] = (uint32_t)(m >> 32);
    n_above += above ? 1u : 0u;
  }
  uint32_t tot_c, tot_a;
  uint32_t slot = block_scan_sum<kMtThreads>(ncand, sc, tot_c);
  block_scan_sum<kMtThreads>(n_above, sc + 8, tot_a);
  const int64_t cb = ((int64_t)row * w.nchunk + chunk);
  if (tid == 0) {
    w.cnt[cb * 2 + 0] = tot_a;
    w.cnt[cb * 2 + 1] = tot_c;
  }
  uint32_t* ck = w.cand_k + cb * kChunkCand;
  uint32_t* cj = w.cand_j + cb * kChunkCand;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = j0 + i * kMtThreads + tid;
    if (j < j1 && ks[i] >= klo && ks[i] <= khi) {
      if (slot < (uint32_t)kChunkCand) {
        ck[slot] = ks[i];
        cj[slot] = j;
      }
      ++slot;
    }
  }
}

struct FinSmem {
  RowSmem row;
  uint32_t ck[kCandCap];
  uint32_t cj[kCandCap];
  uint32_t bm[kMaxWords];
  uint32_t coff[64];
};

__global__ __launch_bounds__(kTkThreads) void mt_finalize_kernel(TopkParams p, MtWs w) {
  constexpr int T = kTkThreads;
  __shared__ FinSmem sm;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  RowCtx c = row_ctx(p, row);
  if (c.n <= p.K) return write_all(p, c, T);
  const int nch = (c.n + kMtChunk - 1) / kMtChunk;
  // per-chunk counts -> offsets (nch <= 64 by construction)
  uint32_t ca = 0, cc = 0;
  bool over = false;
  if (tid < nch) {
    const int64_t cb = (int64_t)row * w.nchunk + tid;
    ca = w.cnt[cb * 2 + 0];
    cc = w.cnt[cb * 2 + 1];
    over = cc > (uint32_t)kChunkCand;
  }
  uint32_t n_above, n_cand;
  const uint32_t coff = block_scan_sum<T>(cc, sm.row.sc, n_cand);
  block_scan_sum<T>(ca, sm.row.sc + 8, n_above);
  if (tid < nch) sm.coff[tid] = coff;
  const bool any_over = __syncthreads_or(over) != 0;
  if (any_over || n_cand > (uint32_t)kCandCap) {   // too many near the threshold: one pass over the row
    row_topk_single<T>(p, c, sm.row);
    if (p.count && tid == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
    return;
  }
  const int nwords = (c.n + 31) >> 5;
  const uint32_t* gb = w.bitmap + (int64_t)row * w.words;
  for (int i = tid; i < nwords; i += T) sm.bm[i] = gb[i];
  for (int ch = 0; ch < nch; ++ch) {
    const uint32_t base = sm.coff[ch];
    const uint32_t num = (ch + 1 < nch ? sm.coff[ch + 1] : n_cand) - base;
    const int64_t cb = ((int64_t)row * w.nchunk + ch) * kChunkCand;
    for (uint32_t i = tid; i < num; i += T) {
      sm.ck[base + i] = w.cand_k[cb + i];
      sm.cj[base + i] = w.cand_j[cb + i];
    }
  }
  __syncthreads();
  uint32_t wlo, whi;
  cand_window(p, c, w.bin[row], wlo, whi);
  const int wbits = 32 - __builtin_clz((whi - wlo) | 1u);
  const uint32_t R = (uint32_t)p.K - n_above;
  uint32_t t, above;
  radix_select<T>((int)n_cand, R, [&](int i, uint32_t& k) { k = sm.ck[i]; return true; }, sm.row.hist,
                  sm.row.sc, t, above, wlo, wbits);
  const float tf = order_key_f32(t);
  uint32_t klo, khi;
  band_limits(p, c, tf, tf, tf, klo, khi);
  // candidates above the band are in; the band goes to a short list
  uint32_t n_in = 0;
  if (tid == 0) sm.row.run[0] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < n_cand; i += T) {
    const uint32_t ks = sm.ck[i];
    if (ks > khi) {
      atomicOr(&sm.bm[sm.cj[i] >> 5], 1u << (sm.cj[i] & 31));
      ++n_in;
    } else if (ks >= klo) {
      const uint32_t slot = atomicAdd(&sm.row.run[0], 1u);
      if (slot < (uint32_t)kBandCap) {
        sm.row.band_j[slot] = sm.cj[i];
        sm.row.band_k[slot] = ks;
      }
    }
  }
  uint32_t tot_in;
  block_scan_sum<T>(n_in, sm.row.sc, tot_in);
  const uint32_t nb = sm.row.run[0];
  const uint32_t R2 = R - tot_in;
  if (nb <= (uint32_t)kBandCap) {
    if (p.certified) {                      // exact keys, one wave per member
      for (uint32_t e = tid >> 6; e < nb; e += T / 64) {
        const float key = wave_exact_key(c.ir, sm.row.band_j[e]);
        if (lane == 0) sm.row.band_k[e] = f32_order_key(key);
      }
      __syncthreads();
    }
    // keep the R2 best by (exact key desc, index asc): rank by counting in the band
    for (uint32_t e = tid; e < nb; e += T) {
      const uint32_t ke = sm.row.band_k[e], je = sm.row.band_j[e];
      uint32_t rank = 0;
      for (uint32_t f = 0; f < nb; ++f) {
        const uint32_t kf = sm.row.band_k[f];
        rank += (kf > ke || (kf == ke && sm.row.band_j[f] < je)) ? 1u : 0u;
      }
      if (rank < R2) atomicOr(&sm.bm[je >> 5], 1u << (je & 31));
    }
  } else {                                  // a very wide band: one thread per member, radix select
    for (uint32_t i = tid; i < n_cand; i += T) {
      const uint32_t ks = sm.ck[i];
      const bool bd = ks >= klo && ks <= khi;
      sm.ck[i] = bd ? exkey_of(p, c, (int)sm.cj[i], ks) : 0u;
      if (bd) sm.cj[i] |= 0x80000000u;
    }
    __syncthreads();
    uint32_t t2, above2;
    radix_select<T>((int)n_cand, R2,
                    [&](int i, uint32_t& k) { k = sm.ck[i]; return (sm.cj[i] & 0x80000000u) != 0; },
                    sm.row.hist, sm.row.sc, t2, above2);
    const uint32_t need_eq = R2 - above2;
    for (uint32_t i = tid; i < n_cand; i += T) {
      if (!(sm.cj[i] & 0x80000000u)) continue;
      const uint32_t j = sm.cj[i] & 0x7FFFFFFFu, k = sm.ck[i];
      bool sel = k > t2;
      if (k == t2) {
        uint32_t rank = 0;
        for (uint32_t f = 0; f < n_cand; ++f)
          rank += ((sm.cj[f] & 0x80000000u) && sm.ck[f] == t2 && (sm.cj[f] & 0x7FFFFFFFu) < j) ? 1u : 0u;
        sel = rank < need_eq;
      }
      if (sel) atomicOr(&sm.bm[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  // bitmap -> ascending indices
  const int per = (nwords + T - 1) / T;
  const int w0 = tid * per, w1 = min(nwords, w0 + per);
  uint32_t cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(sm.bm[i]);
  uint32_t total;
  uint32_t pos = block_scan_sum<T>(cnt, sm.row.sc, total);
  for (int i = w0; i < w1; ++i) {
    uint32_t m = sm.bm[i];
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
  return rows <= 1024 && p.ctx >= 4 * kMtChunk && (p.ctx + 31) / 32 <= kMaxWords &&
         (p.ctx + kMtChunk - 1) / kMtChunk <= 64;
}

size_t topk_ws_bytes(const TopkParams& p) {
  if (!use_multi(p)) return 0;
  const int64_t rows = (int64_t)p.B * p.G * p.Nq;
  const int64_t words = (p.ctx + 31) / 32;
  const int64_t nchunk = (p.ctx + kMtChunk - 1) / kMtChunk;
  return (size_t)rows * (4096 + nchunk * 2 + 1 + words + 2 * nchunk * kChunkCand) * sizeof(uint32_t);
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
  w.cnt = w.hist + (int64_t)rows * 4096;
  w.bin = w.cnt + (int64_t)rows * w.nchunk * 2;
  w.bitmap = w.bin + rows;
  w.cand_k = w.bitmap + (int64_t)rows * w.words;
  w.cand_j = w.cand_k + (int64_t)rows * w.nchunk * kChunkCand;
  hipLaunchKernelGGL(mt_zero_kernel, dim3(rows), dim3(256), 0, st, w);
  hipLaunchKernelGGL(mt_hist_kernel, dim3(w.nchunk, rows), dim3(kMtThreads), 0, st, p, w);
  hipLaunchKernelGGL(mt_collect_kernel, dim3(w.nchunk, rows), dim3(kMtThreads), 0, st, p, w);
  hipLaunchKernelGGL(mt_finalize_kernel, dim3(rows), dim3(kTkThreads), 0, st, p, w);
  return hipGetLastError();
}

}  // namespace sp
