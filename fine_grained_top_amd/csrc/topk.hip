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

// The same for the two-pass kernel, compact: the band lists reuse the
// histogram's storage (the histogram is dead once the threshold is known).
struct RowSmemC {
  union {
    uint32_t hist[4096];
    struct {
      uint32_t band_j[2048];
      uint32_t band_k[2048];
    };
  };
  uint32_t sc[16];
  uint32_t run[4];
};

// A row area whose histogram, once the radix passes are done, holds the band
// lists in its first half and the selected-position bitmap (positions below
// 65536) in its second half.
struct RowSmemF {
  union {
    uint32_t hist[4096];
    struct {
      uint32_t band_j[1024];
      uint32_t band_k[1024];
      uint32_t bm[2048];
    };
  };
  uint32_t sc[16];
  uint32_t run[4];
};

struct RowCtx {
  int b, g, r, n;
  const float* s;
  int32_t* out;
  float eps;             // certified: bound on |score - key| of this row
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
  c.eps = (p.certified && p.err) ? p.err[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] : 0.f;
  if (p.certified) c.ir = indexer_row(p.ix, c.b, c.g, c.r);
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
  const float E = 2.0f * c.eps * 1.0001f + 1e-30f;
  klo = f32_order_key(nextafterf(lo_f - E, -INFINITY));
  khi = f32_order_key(nextafterf(hi_f + E, INFINITY));
  (void)tf;
}

SP_DEV uint32_t exkey_of(const TopkParams& p, const RowCtx& c, int j, uint32_t ks) {
  return p.certified ? f32_order_key(exact_key(c.ir, j)) : ks;
}

// The whole selection for one row by one workgroup of T threads; score(i)
// gives the float32 score of candidate i.
template <int T, typename Score>
SP_DEV void row_topk_single(const TopkParams& p, RowCtx& c, RowSmem& sm, Score score) {
  const int tid = threadIdx.x;
  const int n = c.n, K = p.K;
  auto skey = [&](int i) -> uint32_t { return f32_order_key(score(i)); };
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
  row_topk_single<kTkThreads>(p, c, sm, [&](int i) { return c.s[i]; });
  if (p.count && threadIdx.x == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
}

// Visit s[0..n) as (j, order key), U loads per thread a batch; the next
// batch is in flight while the current one is visited.
template <int T, int U, typename F>
SP_DEV void for_each_key(const float* s, int n, F f) {
  float v[U], w[U];
  auto load = [&](float (&x)[U], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * T + (int)threadIdx.x;
      x[u] = j < n ? s[j] : 0.f;
    }
  };
  load(v, 0);
  for (int base = 0; base < n; base += T * U) {
    const bool more = base + T * U < n;
    if (more) load(w, base + T * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * T + (int)threadIdx.x;
      if (j < n) f(j, f32_order_key(v[u]));
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = w[u];
    }
  }
}

// ---------------------------------------------------------------- two-pass single-workgroup schedule
// Rows of up to 65536 keys: pass 1 builds a 12-bit histogram in LDS and finds
// the bin holding the K-th largest key; pass 2 sets a bitmap bit for every key
// above that bin (plus the certification margin) and lists the keys inside it;
// the short list is resolved exactly and the bitmap is written out in order.
constexpr int kR2Words = 2048;      // bitmap words (65536 keys)
constexpr int kR2Cand = 1860;       // candidates (and samples) kept in LDS
constexpr int kR2Heads = 1;         // indexer heads tracked at once in the exact band keys

// 40 KB, so that four rows run on a CU at once
struct R2Main {
  RowSmemC row;
  float qs[4 * 64];     // certified rows with <= 4 heads of <= 64 dims: queries and weights
  float wsg[4];
  uint32_t ck[kR2Cand];
  uint32_t cj[kR2Cand];
  uint32_t bm[kR2Words];
  uint32_t misc[4];
};
static_assert(sizeof(R2Main) <= 40960, "two-pass top-K shared memory must allow four workgroups per CU");

// Mark in bm the R2 best band members by (exact key desc, position asc). A
// band of at most 64 is ranked by wave 0 from registers (readlane), a larger
// one by every thread from LDS. The caller synchronizes afterwards.
template <int T>
SP_DEV void band_mark(const uint32_t* band_k, const uint32_t* band_j, uint32_t nb, uint32_t R2, uint32_t* bm) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (nb <= 64) {
    if (tid < 64) {
      const uint32_t ke = (uint32_t)lane < nb ? band_k[lane] : 0u;
      const uint32_t je = (uint32_t)lane < nb ? band_j[lane] : 0u;
      uint32_t rank = 0;
      for (uint32_t f = 0; f < nb; ++f) {
        const uint32_t kf = (uint32_t)__builtin_amdgcn_readlane((int)ke, (int)f);
        const uint32_t jf = (uint32_t)__builtin_amdgcn_readlane((int)je, (int)f);
        rank += (kf > ke || (kf == ke && jf < je)) ? 1u : 0u;
      }
      if ((uint32_t)lane < nb && rank < R2) atomicOr(&bm[je >> 5], 1u << (je & 31));
    }
    return;
  }
  for (uint32_t e = tid; e < nb; e += T) {
    const uint32_t ke = band_k[e], je = band_j[e];
    uint32_t rank = 0;
    for (uint32_t f = 0; f < nb; ++f) {
      const uint32_t kf = band_k[f];
      rank += (kf > ke || (kf == ke && band_j[f] < je)) ? 1u : 0u;
    }
    if (rank < R2) atomicOr(&bm[je >> 5], 1u << (je & 31));
  }
}

// Resolve the candidate list (keys ck, indices cj, n_cand of them) that holds
// the remaining R slots; sets the selected bits in bm. Returns false when the
// band is too wide for the short list or an exact band key needs the wide
// accumulator (caller redoes the row).
template <int T, typename SM, int HB = 4, bool SLOW = false, typename CJ = uint32_t>
SP_DEV bool resolve_candidates(const TopkParams& p, RowCtx& c, SM& rs, uint32_t* ck, CJ* cj,
                               uint32_t* bm, uint32_t n_cand, uint32_t R, uint32_t wlo, uint32_t whi,
                               uint32_t tlo = 0u, uint32_t thi = 0xFFFFFFFFu, const float* qs = nullptr,
                               const float* wsg = nullptr, int bm_clear = 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int bits = 32 - __builtin_clz((whi - wlo) | 1u);
  uint32_t t, above;
  radix_select<T>((int)n_cand, R, [&](int i, uint32_t& k) { k = ck[i]; return true; }, rs.hist, rs.sc, t, above,
                  wlo, bits);
  if (t < tlo || t > thi) return false;   // the band might reach past the window
  const float tf = order_key_f32(t);
  uint32_t klo, khi;
  band_limits(p, c, tf, tf, tf, klo, khi);
  uint32_t n_in = 0;
  // a bitmap that shares the histogram's memory is cleared only now
  for (int i = tid; i < bm_clear; i += T) bm[i] = 0u;
  if (tid == 0) rs.run[0] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < n_cand; i += T) {
    const uint32_t ks = ck[i], js = (uint32_t)cj[i];
    if (ks > khi) {
      atomicOr(&bm[js >> 5], 1u << (js & 31));
      ++n_in;
    } else if (ks >= klo) {
      const uint32_t slot = atomicAdd(&rs.run[0], 1u);
      if (slot < (uint32_t)(sizeof(rs.band_j) / sizeof(uint32_t))) {
        rs.band_j[slot] = js;
        rs.band_k[slot] = ks;
      }
    }
  }
  uint32_t tot_in;
  block_scan_sum<T>(n_in, rs.sc, tot_in);
  const uint32_t nb = rs.run[0];
  if (nb > (uint32_t)(sizeof(rs.band_j) / sizeof(uint32_t))) return false;
  const uint32_t R2 = R - tot_in;
  if (p.certified) {
    if (tid == 0) rs.run[1] = 0;
    __syncthreads();
    for (uint32_t e = tid >> 4; e < nb; e += T / 16) {   // a quarter-wave per band member
      const float key = group_exact_key<16, HB, SLOW>(c.ir, rs.band_j[e], qs, wsg);
      if ((lane & 15) == 0) {
        rs.band_k[e] = f32_order_key(key);
        if (key != key) rs.run[1] = 1u;             // not settled without the wide accumulator
      }
    }
    __syncthreads();
    if (rs.run[1]) return false;
  }
  band_mark<T>(rs.band_k, rs.band_j, nb, R2, bm);
  __syncthreads();
  return true;
}

// Write the set bits of bm (nwords <= MAXW words) as ascending indices, pad
// with -1. Thread t owns a contiguous run of words, read from LDS once.
template <int T, int MAXW, typename SM>
SP_DEV void emit_bitmap(const TopkParams& p, const RowCtx& c, SM& rs, const uint32_t* bm, int nwords) {
  constexpr int PW = (MAXW + T - 1) / T;
  const int tid = threadIdx.x;
  const int perw = (nwords + T - 1) / T;
  const int w0 = tid * perw;
  uint32_t wv[PW];
  uint32_t cnt = 0;
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    wv[q] = (q < perw && w0 + q < nwords) ? bm[w0 + q] : 0u;
    cnt += __popc(wv[q]);
  }
  uint32_t total;
  uint32_t pos = block_scan_sum<T>(cnt, rs.sc, total);
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    uint32_t m = wv[q];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (pos < (uint32_t)p.K) c.out[pos] = (w0 + q) * 32 + bit;
      ++pos;
    }
  }
  for (int i = (int)total + tid; i < p.K; i += T) c.out[i] = -1;
  if (p.count && tid == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = (int)min(total, (uint32_t)p.K);
}

// Order-key window [tlo, thi] that holds the rhi-th and the rlo-th largest of
// the valid keys in k[0..m) (order key 0 marks an unused slot; rhi <= rlo <=
// number of valid keys). A 4096-bin histogram over the keys' range gives the
// bins of the two ranks; a second histogram over the span of those bins
// refines them (a wide range, e.g. with ReLU zeros, would otherwise leave
// bins far coarser than the rank window). thi is the upper edge of the final
// bin of rank rhi, tlo the lower edge of the final bin of rank rlo.
template <int T>
SP_DEV void sample_window(const uint32_t* k, int m, uint32_t rhi, uint32_t rlo, uint32_t* hist, uint32_t* sc,
                          uint32_t& tlo, uint32_t& thi) {
  constexpr int NW = T / 64;
  constexpr int per = 4096 / T;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = tid; i < m; i += T) {
    const uint32_t v = k[i];
    if (v != 0u) {
      kmin = min(kmin, v);
      kmax = max(kmax, v);
    }
  }
  kmin = ~wave_max_u32_dpp(~kmin);
  kmax = wave_max_u32_dpp(kmax);
  if (lane == 0) {
    sc[wid] = kmin;
    sc[NW + wid] = kmax;
  }
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, sc[w]);
    hi = max(hi, sc[NW + w]);
  }
  uint32_t above = 0;      // valid keys above hi (none at the first level)
  for (int level = 0; level < 2; ++level) {
    __syncthreads();
    for (int i = tid; i < 4096; i += T) hist[i] = 0u;
    __syncthreads();
    const int bits = 32 - __builtin_clz((hi - lo) | 1u);
    const int sh = bits > 12 ? bits - 12 : 0;
    for (int i = tid; i < m; i += T) {
      const uint32_t v = k[i];
      if (v != 0u && v >= lo && v <= hi) atomicAdd(&hist[(v - lo) >> sh], 1u);
    }
    __syncthreads();
    // counts from the top: thread tid owns bins [per tid, per tid + per)
    uint32_t hb[per], cnt = 0;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      hb[e] = hist[per * tid + e];
      cnt += hb[e];
    }
    uint32_t tot;
    const uint32_t below = block_scan_sum<T>(cnt, sc, tot);
    uint32_t acc = above + tot - below - cnt;
    uint32_t* res = hist;   // results, once every thread has read its bins
    __syncthreads();
#pragma unroll
    for (int e = per - 1; e >= 0; --e) {
      const uint32_t nxt = acc + hb[e];
      const uint32_t bin = (uint32_t)(per * tid + e);
      if (acc < rhi && rhi <= nxt) {
        res[0] = (uint32_t)min((uint64_t)hi, (uint64_t)lo + (((uint64_t)bin + 1) << sh) - 1);
        res[2] = acc;                          // keys above that bin
      }
      if (acc < rlo && rlo <= nxt) res[1] = lo + (bin << sh);
      acc = nxt;
    }
    __syncthreads();
    const uint32_t nhi = res[0], nlo = res[1], nab = res[2];
    if (sh == 0 || level == 1) {
      thi = nhi;
      tlo = nlo;
      break;
    }
    hi = nhi;
    lo = nlo;
    above = nab;
  }
  __syncthreads();
}

constexpr int kR2Threads = 256;

// One row of up to 65536 keys (see above). SLOW = false keeps the function
// within 128 registers (four rows per CU): exact band keys one indexer head at
// a time, no wide accumulator (a key it would need fails the row). Returns
// false when the row needs the ordered single-pass routine (a window that
// misses the threshold, too many keys near it, or such a key).
template <bool SLOW>
SP_DEV bool row2_select(const TopkParams& p, int row, R2Main& sm) {
  constexpr int T = kR2Threads;
  RowCtx c = row_ctx(p, row);
  const int tid = threadIdx.x;
  if (c.n <= p.K) {
    write_all(p, c, T);
    return true;
  }
  const int n = c.n;
  const int nwords = (n + 31) >> 5;
  const uint32_t K = (uint32_t)p.K;
  // certified rows: the row's queries and weights into LDS for the exact band keys
  const bool staged = p.certified && c.ir.H <= 4 && c.ir.d <= 64;
  if (staged) {
    for (int e = tid; e < c.ir.H * c.ir.d; e += T)
      sm.qs[e] = (float)load_f64(c.ir.q, c.ir.qt, (e / c.ir.d) * c.ir.qh_stride + e % c.ir.d);
    if (tid < c.ir.H) sm.wsg[tid] = c.ir.relu ? c.ir.w[tid * c.ir.w_stride] : 1.f;
  }
  const float* qsp = staged ? sm.qs : nullptr;
  const float* wsp = staged ? sm.wsg : nullptr;

  // pass 2 for a window [wlo, whi] (order keys, already widened by the band):
  // bitmap of the keys above it, short list of the keys inside it, exact
  // resolution; false when the window does not hold the threshold with its
  // band (t must lie in [tlo, thi]) or the list overflows
  auto pass2 = [&](uint32_t wlo, uint32_t whi, uint32_t tlo, uint32_t thi) -> bool {
    for (int i = tid; i < nwords; i += T) sm.bm[i] = 0;
    if (tid == 0) sm.misc[0] = 0;
    __syncthreads();
    uint32_t n_above = 0;
    for_each_key<T, 8>(c.s, n, [&](int j, uint32_t ks) {
      if (ks > whi) {
        atomicOr(&sm.bm[j >> 5], 1u << (j & 31));
        ++n_above;
      } else if (ks >= wlo) {
        const uint32_t slot = atomicAdd(&sm.misc[0], 1u);
        if (slot < (uint32_t)kR2Cand) {
          sm.ck[slot] = ks;
          sm.cj[slot] = j;
        }
      }
    });
    uint32_t tot_above;
    block_scan_sum<T>(n_above, sm.row.sc, tot_above);
    const uint32_t n_cand = sm.misc[0];
    if (n_cand > (uint32_t)kR2Cand || tot_above >= K || tot_above + n_cand < K) return false;
    // one indexer head at a time in the exact band keys: the kernel stays
    // within 128 registers (four rows per CU) without spilling
    return resolve_candidates<T, RowSmemC, SLOW ? 4 : kR2Heads, SLOW>(p, c, sm.row, sm.ck, sm.cj, sm.bm, n_cand,
                                                                       K - tot_above, wlo, whi, tlo, thi, qsp, wsp);
  };

  // pass 1, sampled: runs of 64 keys every S (all keys when n <= 1856); the
  // window is the sample's order statistics around the expected rank of the
  // K-th key, with a margin of a few standard deviations
  {
    const int S = 64 * ((n + 1855) / 1856);
    const int nruns = (n + S - 1) / S;
    const int m_all = nruns * 64;                  // <= 1856 slots
    uint32_t mloc = 0;
    for (int e0 = 0; e0 < m_all; e0 += 8 * T) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * T + tid;
        const int j = (e >> 6) * S + (e & 63);
        v[u] = (e < m_all && j < n) ? c.s[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * T + tid;
        const int j = (e >> 6) * S + (e & 63);
        const bool ok = e < m_all && j < n;
        if (e < m_all) sm.ck[e] = ok ? f32_order_key(v[u]) : 0u;
        mloc += ok ? 1u : 0u;
      }
    }
    uint32_t m;
    block_scan_sum<T>(mloc, sm.row.sc, m);        // (its barriers also publish the samples)
    uint32_t rhi, rlo;
    if ((int)m == n) {
      rhi = rlo = K;                              // the sample is the row: exact ranks
    } else {
      // 2.5 standard deviations of the sample rank, but no wider than what
      // keeps the expected number of candidates at 70 % of the list
      const float r = (float)K * (float)m / (float)n;
      const float dlt = fminf(2.5f * sqrtf(r) + 2.f, 0.35f * (float)kR2Cand * (float)m / (float)n);
      rhi = (uint32_t)fmaxf(1.f, floorf(r - dlt));
      rlo = (uint32_t)fminf((float)m, ceilf(r + dlt));
    }
    uint32_t thi, tlo;
    sample_window<T>(sm.ck, m_all, rhi, rlo, sm.row.hist, sm.row.sc, tlo, thi);
    uint32_t wlo, whi;
    band_limits(p, c, 0.f, order_key_f32(tlo), order_key_f32(thi), wlo, whi);
    __syncthreads();
    if (pass2(wlo, whi, tlo, thi)) {
      emit_bitmap<T, kR2Words>(p, c, sm.row, sm.bm, nwords);
      return true;
    }
    __syncthreads();
  }

  // pass 1, full: histogram of the top 12 bits; the window is the bin of the
  // K-th key widened by the band
  for (int i = tid; i < 4096; i += T) sm.row.hist[i] = 0;
  __syncthreads();
  for_each_key<T, 8>(c.s, n, [&](int j, uint32_t ks) { atomicAdd(&sm.row.hist[ks >> 20], 1u); });
  __syncthreads();
  uint32_t bin;
  {
    constexpr int per = 4096 / T;
    const int lo = tid * per;
    uint32_t mine = 0;
    for (int q = 0; q < per; ++q) mine += sm.row.hist[lo + q];
    uint32_t tot;
    const uint32_t below = block_scan_sum<T>(mine, sm.row.sc, tot);
    uint32_t cum = tot - below - mine;
    if (cum < K && cum + mine >= K) {
      for (int q = per - 1; q >= 0; --q) {
        if (cum + sm.row.hist[lo + q] >= K) {
          sm.misc[1] = (uint32_t)(lo + q);
          break;
        }
        cum += sm.row.hist[lo + q];
      }
    }
    __syncthreads();
    bin = sm.misc[1];
  }
  uint32_t wlo, whi;
  {
    const float lo_b = order_key_f32(bin << 20), hi_b = order_key_f32((bin << 20) | 0xFFFFFu);
    band_limits(p, c, 0.f, lo_b, hi_b, wlo, whi);
  }
  __syncthreads();
  if (!pass2(wlo, whi, bin << 20, (bin << 20) | 0xFFFFFu)) return false;
  emit_bitmap<T, kR2Words>(p, c, sm.row, sm.bm, nwords);
  return true;
}

// Rows of up to 65536 keys, one workgroup each: 256 threads held to 128
// registers, 40 KB of LDS, four rows per CU. A row that this kernel cannot
// finish is only flagged in redo[row] (the rare paths would cost every row
// registers); topk_redo_kernel finishes it.
__global__ __launch_bounds__(kR2Threads) __attribute__((amdgpu_waves_per_eu(4))) void topk_row2_kernel(TopkParams p,
                                                                                                      uint32_t* redo) {
  __shared__ R2Main sm;
  const bool done = row2_select<false>(p, blockIdx.x, sm);
  if (threadIdx.x == 0) redo[blockIdx.x] = done ? 0u : 1u;
}

// Rows flagged by topk_row2_kernel: each workgroup takes blocks of kR2Threads
// rows, reads their flags with one load per thread, lists the flagged ones in
// LDS and redoes each with the wide exact accumulator available, then, if
// that fails too, with the ordered single-pass routine.
union R2Redo {
  R2Main m;
  RowSmem full;
};
constexpr int kRedoGrid = 256;
__global__ __launch_bounds__(kR2Threads) void topk_redo_kernel(TopkParams p, const uint32_t* redo, int rows) {
  __shared__ R2Redo smu;
  __shared__ uint32_t list[kR2Threads];
  __shared__ uint32_t nlist;
  for (int r0 = blockIdx.x * kR2Threads; r0 < rows; r0 += gridDim.x * kR2Threads) {
    if (threadIdx.x == 0) nlist = 0u;
    __syncthreads();
    const int row = r0 + (int)threadIdx.x;
    if (row < rows && redo[row] != 0u) list[atomicAdd(&nlist, 1u)] = (uint32_t)row;
    __syncthreads();
    const uint32_t nl = nlist;
    for (uint32_t q = 0; q < nl; ++q) {
      const int rq = (int)list[q];
      if (!row2_select<true>(p, rq, smu.m)) {
        __syncthreads();
        RowCtx c = row_ctx(p, rq);
        row_topk_single<kR2Threads>(p, c, smu.full, [&](int i) { return c.s[i]; });
        if (p.count && threadIdx.x == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
      }
      __syncthreads();
    }
  }
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
  for_each_key<kMtThreads, 16>(c.s + j0, j1 - j0, [&](int, uint32_t ks) { atomicAdd(&h[ks >> 20], 1u); });
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
    row_topk_single<T>(p, c, sm.row, [&](int i) { return c.s[i]; });
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

// ---------------------------------------------------------------- fused indexer + top-K
// The score matrix is never written. A pilot scores a sample of each row's
// keys (runs of 64 keys at a fixed stride) and sets a threshold tau whose
// expected number of survivors is about 1.5 K; the MFMA indexer then keeps
// only (key, index) pairs with score >= tau; the finalize kernel selects the
// exact top-K among them (certified, as above) after checking that every key
// that could belong to it was kept (count >= K and t - 2 eps >= tau). When a
// check fails the row is redone by recomputing scores, so the result never
// depends on the sample.
constexpr int kPilotStride = 2048, kPilotRun = 64, kPilotCap = 8192;
// the decode pilot's sample (few rows: the pilot's span is set by the keys
// one workgroup scores): runs of 64 keys every 8192
constexpr int kDecStride = 8192, kDecRun = 64, kDecCap = 4096;

// float32 score recomputed by one thread (FMA chains; within the same bound)
SP_DEV float recompute_score(const IndexerRow& r, int64_t j) {
  const int64_t koff = j * r.k_stride;
  float s = 0.f;
  for (int h = 0; h < r.H; ++h) {
    float d = 0.f;
    for (int c = 0; c < r.d; ++c)
      d = fmaf((float)load_f64(r.q, r.qt, h * r.qh_stride + c), (float)load_f64(r.k, r.kt, koff + c), d);
    s = r.relu ? fmaf(r.w[h * r.w_stride], fmaxf(d, 0.f), s) : d;
  }
  return s;
}

// The same float32 score with the row's queries and weights already in LDS
// (qs [H][d], wsg [H]) and the key read four elements per load.
SP_DEV float recompute_score_lds(const IndexerRow& r, const float* qs, const float* wsg, int64_t j) {
  const int64_t koff = j * r.k_stride;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < r.d; c += 4) {
    double kv[4];
    load_run_f64<4>(r.k, r.kt, koff + c, r.d - c, kv);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (h < r.H)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < r.d) acc[h] = fmaf(qs[h * r.d + c + e], (float)kv[e], acc[h]);
  }
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h)
    if (h < r.H) s = r.relu ? fmaf(wsg[h], fmaxf(acc[h], 0.f), s) : acc[h];
  return s;
}

// Pilot: one workgroup per selection row. The row's heads score a 1/128
// sample of its keys (runs of 64 keys every 8192) on MFMA, laid out as in
// the indexer (32x32x16 bf16: A = the row's heads as slot rows, B = 32 keys,
// fp8 keys converted to bf16 exactly), so lanes 0..31 each hold every head's
// product for one key and form its score in-lane. The order keys stay in
// LDS; tau is the lower edge of the 4096-bin histogram bin (over the range of
// the sampled keys) where about 1.5 K survivors in proportion (plus 8
// sampled keys) are reached. Any tau is correct: the final
// stage checks it and can fall back; this one only has to leave a little
// over 1.5 K keys. Requires d_I = 64, bf16 queries, bf16 or fp8 keys.
constexpr int kPilotTB = 8;       // sampled tiles of 32 keys per wave and load batch
__global__ __launch_bounds__(kTkThreads) void fz_pilot_kernel(TopkParams p, float* tau) {
  constexpr int T = kTkThreads;
  constexpr int NW = T / 64;
  __shared__ uint32_t sk[kDecCap];
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t sc[16];
  __shared__ uint32_t red[2 * NW + 2];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  RowCtx c = row_ctx(p, row);
  if (c.n <= p.K) {
    if (tid == 0) tau[row] = INFINITY;   // every key is selected; nothing to filter
    return;
  }
  const IndexerRow& ir = c.ir;
  const int nruns = (c.n + kDecStride - 1) / kDecStride;
  const int ntiles = 2 * nruns;                  // two tiles of 32 keys per run
  const int slots = nruns * kDecRun;
  const bool fp8 = ir.kt == DT_FP8;
  // A operand: slot row col = head col (< H), dims 32 half + 8 s + v
  bf16x8 A[4];
  if (col < ir.H) {
    const uint16_t* qp = (const uint16_t*)ir.q + col * ir.qh_stride + 32 * half;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) A[s4] = *(const bf16x8*)(qp + 8 * s4);
  } else {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) A[s4] = (bf16x8){};
  }
  float wv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) wv[t] = (ir.relu && t < ir.H) ? ir.w[t * ir.w_stride] : 0.f;
  const int tbstep = NW * (fp8 ? kPilotTB : kPilotTB / 2);
  for (int tb = wid; tb < ntiles; tb += tbstep) {
    // key bytes of this wave's batch: tile tt = tb + NW u covers keys
    // (tt / 2) * 8192 + 32 (tt % 2) + col, lane half: dims 32 half .. +31
    u32x4 raw[kPilotTB][4];
#pragma unroll
    for (int u = 0; u < kPilotTB; ++u) {
      const int tt = tb + NW * u;
      int j = (tt >> 1) * kDecStride + 32 * (tt & 1) + col;
      j = j < c.n ? j : c.n - 1;
      if (tt < ntiles) {
        if (fp8) {
          const u32x4* kp = (const u32x4*)((const uint8_t*)ir.k + (int64_t)j * ir.k_stride + 32 * half);
          raw[u][0] = kp[0];
          raw[u][1] = kp[1];
        } else if (u < kPilotTB / 2) {           // bf16 rows are twice as long: half the batch
          const u32x4* kp = (const u32x4*)((const uint16_t*)ir.k + (int64_t)j * ir.k_stride + 32 * half);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) raw[u][q4] = kp[q4];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPilotTB; ++u) {
      const int tt = tb + NW * u;
      if (tt >= ntiles || (!fp8 && u >= kPilotTB / 2)) continue;
      u32x4 Bw[4];
      if (fp8) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const uint32_t w0 = raw[u][s4 >> 1][2 * (s4 & 1)], w1 = raw[u][s4 >> 1][2 * (s4 & 1) + 1];
          Bw[s4][0] = fp8x2_to_bf16x2<false>(w0);
          Bw[s4][1] = fp8x2_to_bf16x2<true>(w0);
          Bw[s4][2] = fp8x2_to_bf16x2<false>(w1);
          Bw[s4][3] = fp8x2_to_bf16x2<true>(w1);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) Bw[s4] = raw[u][s4];
      }
      f32x16 acc = {};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s4], *(const bf16x8*)&Bw[s4], acc, 0, 0, 0);
      // lanes of half 0 hold slot rows 0..3 (the heads) of key col
      float sv = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        sv = ir.relu ? fmaf(wv[t], __int_as_float(max(__float_as_int(acc[t]), 0)), sv) : acc[0];
      const int j = (tt >> 1) * kDecStride + 32 * (tt & 1) + col;
      if (half == 0) sk[32 * tt + col] = j < c.n ? f32_order_key(sv) : 0u;
    }
  }
  __syncthreads();
  // tau from the sampled keys (0 marks a key after the row's position)
  constexpr int U = kDecCap / T;
  uint32_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = tid + u * T;
    v[u] = i < slots ? sk[i] : 0u;
  }
  for (int i = tid; i < 4096; i += T) hist[i] = 0u;
  uint32_t m = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (v[u] != 0u) {
      ++m;
      kmin = min(kmin, v[u]);
      kmax = max(kmax, v[u]);
    }
  m = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl_u32(m), 63);
  kmin = ~wave_max_u32_dpp(~kmin);
  kmax = wave_max_u32_dpp(kmax);
  if (lane == 0) {
    red[wid] = kmin;
    red[NW + wid] = kmax;
    sc[wid] = m;
  }
  __syncthreads();
  uint32_t mt = 0;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
  for (int x = 0; x < NW; ++x) {
    mt += sc[x];
    kmin = min(kmin, red[x]);
    kmax = max(kmax, red[NW + x]);
  }
  __syncthreads();                                          // sc is reused by the scan below
  const uint64_t want = ((uint64_t)3 * p.K * mt + 2ull * c.n - 1) / (2ull * c.n) + 8;   // ~1.5 K survivors
  const uint32_t R = (uint32_t)min((uint64_t)mt, want);
  if (R == 0) {
    if (tid == 0) tau[row] = -INFINITY;
    return;
  }
  const int bits = 32 - __builtin_clz((kmax - kmin) | 1u);
  const int sh = bits > 12 ? bits - 12 : 0;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (v[u] != 0u) atomicAdd(&hist[(v[u] - kmin) >> sh], 1u);
  __syncthreads();
  // count from the top: thread tid owns bins [8 tid, 8 tid + 8)
  uint32_t hb[8], cnt = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hb[e] = hist[8 * tid + e];
    cnt += hb[e];
  }
  uint32_t tot;
  const uint32_t below = block_scan_sum<T>(cnt, sc, tot);   // members in lower threads' bins
  const uint32_t above0 = tot - below - cnt;                // members in higher threads' bins
  if (above0 < R && R <= above0 + cnt) {
    uint32_t acc = above0;
    int bin = 8 * tid;
    for (int e = 7; e >= 0; --e) {
      acc += hb[e];
      if (acc >= R) {
        bin = 8 * tid + e;
        break;
      }
    }
    tau[row] = order_key_f32(kmin + ((uint32_t)bin << sh));
  }
}

struct FzWs {
  float* tau;
  float* kmax;
  uint32_t* cand_n;
  u32x2* cand;             // (order key, key position) pairs
  int nchunk, cap;
};

constexpr int kFzOvf = 1024;

struct FzSmem {
  RowSmem row;             // histogram and band lists (also used by the fallback)
  uint32_t bm[kMaxWords];
  float qs[4 * 64];        // the row's indexer queries (<= 4 heads, d_I = 64) and weights
  float wsg[4];
  float red[4 * (kTkThreads / 64)];   // per-wave partials
  u32x2 ovf[kFzOvf];       // candidate slots past the first 32 of a chunk, per wave, read once
  uint32_t ovn[kTkThreads / 64];   // entries of each wave's region (all ones: it did not fit)
};

// In a 4096-bin histogram (bins ordered low to high), the bin holding the
// R-th largest element and the number of elements in higher bins. Thread t
// owns bins [8t, 8t + 8). Two barriers; hist may be rewritten afterwards.
template <int T>
SP_DEV void hist_find(const uint32_t* hist, uint32_t R, uint32_t* sc, uint32_t& bin, uint32_t& above) {
  static_assert(T * 8 == 4096, "eight bins per thread");
  constexpr int NW = T / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t hb[8], mine = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hb[e] = hist[8 * tid + e];
    mine += hb[e];
  }
  const uint32_t pin = wave_prefix_incl_u32(mine);
  const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)pin, 63) - pin + mine;   // this lane and above
  if (lane == 0) sc[wid] = v;
  __syncthreads();
  uint32_t cum = v - mine;
#pragma unroll
  for (int x = 0; x < NW; ++x) cum += x > wid ? sc[x] : 0u;
  if (cum < R && cum + mine >= R) {
#pragma unroll
    for (int e = 7; e >= 0; --e) {
      if (cum + hb[e] >= R) {
        sc[NW] = (uint32_t)(8 * tid + e);
        sc[NW + 1] = cum;
        break;
      }
      cum += hb[e];
    }
  }
  __syncthreads();
  bin = sc[NW];
  above = sc[NW + 1];
}

// first-round reads of the final selection: 16 lanes per chunk, one 16-byte
// pair of candidate slots each (the first 32 slots of 32 chunks per
// instruction); slots past 32 of a chunk are read from global memory in
// every pass (a chunk rarely holds that many)
constexpr int kFzLanes = 16;
constexpr int kFzRounds = 8;      // instructions held in registers: 256 chunks

// Final selection, one workgroup per row. Every load of the row is issued in
// one round, none waiting on another: the first 32 candidate slots of every
// chunk (consecutive lanes read consecutive pairs of a chunk's slots) with
// the chunk counts, the chunk key bounds, the threshold, the row's queries
// and weights; a thread whose chunk holds more reads the rest into its
// wave's LDS list. Each thread counts its candidates and their largest score
// on the way, so one barrier publishes the error bound's inputs, the number
// of candidates and the largest score. The K-th largest score is located by
// a histogram of 4096 bins over [tau, largest score] (bins as wide as the
// certification band or wider; a second pass splits the bin when it is much
// wider); the band is that bin's range widened by the certification margin;
// scores above it set bitmap bits, band members are listed and, unless all
// of them are needed to fill the K slots, scored exactly and ranked; the
// bitmap is written out as ascending positions. Checks (enough candidates,
// the band above tau) send a row to recomputed scores, so the result never
// depends on the pilot's sample.
__global__ __launch_bounds__(kTkThreads) void fz_final_kernel(TopkParams p, FzWs w) {
  constexpr int T = kTkThreads, NW = T / 64, S = kFzRounds, CPI = T / kFzLanes;
  __shared__ FzSmem sm;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nrl = p.G * p.Nq, rowl = row % nrl, b = row / nrl;
  const int cq = tid / kFzLanes, pr = tid % kFzLanes;     // chunk within an instruction, slot pair
  // candidate slots of chunk ch for this row; counts
  auto cslot = [&](int ch) { return w.cand + (((int64_t)b * w.nchunk + ch) * nrl + rowl) * w.cap; };
  auto ccount = [&](int ch) { return w.cand_n[((int64_t)b * w.nchunk + ch) * nrl + rowl]; };
  u32x4 cv4[S];
  uint32_t cn[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int ch = CPI * i + cq;
    if (ch < w.nchunk) {
      cv4[i] = ((const u32x4*)cslot(ch))[pr];
      cn[i] = ccount(ch);
    }
  }
  float km = tid < w.nchunk ? w.kmax[(int64_t)b * w.nchunk + tid] : 0.f;
  const float tau = w.tau[row];
  RowCtx c = row_ctx(p, row);
  const int H = c.ir.H, d = c.ir.d;
  float qv = 0.f, wq = 0.f;
  if (tid < H * d) {
    qv = (float)load_f64(c.ir.q, c.ir.qt, (tid / d) * c.ir.qh_stride + tid % d);
    wq = c.ir.relu ? c.ir.w[(tid / d) * c.ir.w_stride] : 1.f;
  }
  if (c.n <= p.K) return write_all(p, c, T);
  if (tid < H * d) sm.qs[tid] = qv;
  if (tid < H * d && tid % d == 0) sm.wsg[tid / d] = wq;
  float coef = tid < H * d ? fabsf(wq) * fabsf(qv) : 0.f;
  const int nch = (c.n + 511) / 512;                 // chunks holding keys 0..n-1
  if (tid >= nch) km = 0.f;
  // register pairs: bit 2 i + h set when entry h of pair i is a candidate
  uint32_t vm = 0u;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int ch = CPI * i + cq;
    const uint32_t nn = ch < nch ? min(cn[i], 32u) : 0u;
    vm |= ((uint32_t)(2 * pr) < nn ? 1u : 0u) << (2 * i);
    vm |= ((uint32_t)(2 * pr + 1) < nn ? 1u : 0u) << (2 * i + 1);
  }
  // visit every candidate of this thread: register pairs, then (rare) the
  // slots past 32 of this thread's chunks and the chunks past the registers
  bool xs = false;                                     // a register chunk holds more than 32
#pragma unroll
  for (int i = 0; i < S; ++i) xs |= CPI * i + cq < nch && cn[i] > 32u;
  // The slots past 32 of the register chunks are read once, by the thread
  // that owns them, into its wave's region of an LDS list (the wave's
  // offsets from a prefix sum of the per-thread counts); every pass below
  // visits the list. A wave whose slots exceed its region reads them from
  // global memory in every pass instead.
  constexpr int kOvfW = kFzOvf / (T / 64);
  uint32_t nov = 0u;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int ch = CPI * i + cq;
    const int lim = ch < nch ? (int)min(cn[i], (uint32_t)w.cap) : 0;
    if (lim > 32 + pr) nov += (uint32_t)((lim - 32 - pr + kFzLanes - 1) / kFzLanes);
  }
  const uint32_t ov_incl = wave_prefix_incl_u32(nov);
  const uint32_t ov_wave = (uint32_t)__builtin_amdgcn_readlane((int)ov_incl, 63);
  const bool ov_fit = ov_wave <= (uint32_t)kOvfW;
  // the counting pass: this thread's candidates (registers, its slots past
  // 32, the chunks past the registers)
  uint32_t kmx = 0u, mine = 0u;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    if (vm & (1u << (2 * i))) { kmx = max(kmx, cv4[i][0]); ++mine; }
    if (vm & (2u << (2 * i))) { kmx = max(kmx, cv4[i][2]); ++mine; }
  }
  if (xs) {
    uint32_t o = (uint32_t)wid * kOvfW + ov_incl - nov;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int ch = CPI * i + cq;
      if (ch < nch && cn[i] > 32u)
        for (int e = 32 + pr; e < (int)min(cn[i], (uint32_t)w.cap); e += kFzLanes) {
          const u32x2 v = cslot(ch)[e];
          kmx = max(kmx, v[0]);
          ++mine;
          if (ov_fit) sm.ovf[o++] = v;
        }
    }
  }
  for (int ch = CPI * S + cq; ch < nch; ch += CPI) {   // chunks past the registers (long contexts)
    const int nn = (int)min(ccount(ch), (uint32_t)w.cap);
    for (int e = pr; e < nn; e += kFzLanes) {
      kmx = max(kmx, cslot(ch)[e][0]);
      ++mine;
    }
  }
  if (lane == 0) sm.ovn[wid] = ov_fit ? ov_wave : 0xFFFFFFFFu;
  bool ovf_lds = true;                                 // set after the barrier below
  auto each = [&](auto f) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      if (vm & (1u << (2 * i))) f(cv4[i][0], cv4[i][1]);
      if (vm & (2u << (2 * i))) f(cv4[i][2], cv4[i][3]);
    }
    if (ovf_lds) {
#pragma unroll
      for (int v = 0; v < T / 64; ++v)
        for (uint32_t e = tid; e < sm.ovn[v]; e += T) {
          const u32x2 x = sm.ovf[v * kOvfW + e];
          f(x[0], x[1]);
        }
    } else if (xs) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const int ch = CPI * i + cq;
        if (ch < nch && cn[i] > 32u)
          for (int e = 32 + pr; e < (int)min(cn[i], (uint32_t)w.cap); e += kFzLanes) {
            const u32x2 v = cslot(ch)[e];
            f(v[0], v[1]);
          }
      }
    }
    for (int ch = CPI * S + cq; ch < nch; ch += CPI) {   // chunks past the registers (long contexts)
      const int nn = (int)min(ccount(ch), (uint32_t)w.cap);
      for (int e = pr; e < nn; e += kFzLanes) {
        const u32x2 v = cslot(ch)[e];
        f(v[0], v[1]);
      }
    }
  };
  bool over = false;
#pragma unroll
  for (int i = 0; i < S; ++i) over |= CPI * i + cq < nch && cn[i] > (uint32_t)w.cap;
  for (int i = tid; i < 4096; i += T) sm.row.hist[i] = 0u;
  const int nwords = (c.n + 31) >> 5;
  for (int i = tid; i < nwords; i += T) sm.bm[i] = 0u;
  if (tid == 0) {
    sm.row.run[0] = 0u;
    sm.row.run[1] = 0u;
  }
  km = wave_max_dpp(km);
  coef = wave_sum_dpp(coef);
  kmx = wave_max_u32_dpp(kmx);
  const uint32_t wn = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl_u32(mine), 63);
  const bool wover = __any(over);
  if (lane == 0) {
    sm.red[wid] = km;
    sm.red[NW + wid] = coef;
    sm.red[2 * NW + wid] = __uint_as_float(kmx);
    sm.red[3 * NW + wid] = __uint_as_float(wn | (wover ? 0x80000000u : 0u));
  }
  __syncthreads();
  float KM = 0.f, CO = 0.f;
  uint32_t KX = 0u, n_cand = 0u;
  bool any_over = false;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    KM = fmaxf(KM, sm.red[v]);
    CO += sm.red[NW + v];
    KX = max(KX, __float_as_uint(sm.red[2 * NW + v]));
    const uint32_t x = __float_as_uint(sm.red[3 * NW + v]);
    n_cand += x & 0x7FFFFFFFu;
    any_over |= (x >> 31) != 0u;
  }
#pragma unroll
  for (int v = 0; v < NW; ++v) ovf_lds &= sm.ovn[v] != 0xFFFFFFFFu;
  c.eps = eps_of(p.ix, CO, KM);
  auto fallback = [&]() {
    row_topk_single<T>(p, c, sm.row, [&](int i) { return recompute_score(c.ir, i); });
    if (p.count && tid == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
  };
  if (any_over || n_cand < (uint32_t)p.K || !(fabsf(tau) <= 3.0e38f)) return fallback();
  const float E = 2.0f * c.eps * 1.0001f + 1e-30f;            // half-width of the band
  // bins of [tau, largest score]: bin(s) = floor((s - tau) / W), monotone in s
  const float W = fmaxf(E, (order_key_f32(KX) - tau) * (1.0f / 4096.0f) * 1.001f);
  const float iW = 1.0f / W;
  auto bin1 = [&](uint32_t k) { return (uint32_t)fminf((order_key_f32(k) - tau) * iW, 4095.0f); };
  each([&](uint32_t k, uint32_t) { atomicAdd(&sm.row.hist[bin1(k)], 1u); });
  __syncthreads();
  uint32_t b1, above;
  hist_find<T>(sm.row.hist, (uint32_t)p.K, sm.row.sc, b1, above);
  // a bin much wider than the band: split it into 4096 once more
  const bool two = W > 4.0f * E;
  uint32_t b2 = 0u;
  const float lo2 = tau + (float)b1 * W, iW2 = 4096.0f / (W * 1.01f);
  auto bin2 = [&](uint32_t k) { return (uint32_t)fminf(fmaxf((order_key_f32(k) - lo2) * iW2, 0.0f), 4095.0f); };
  if (two) {
    for (int i = tid; i < 4096; i += T) sm.row.hist[i] = 0u;
    __syncthreads();
    each([&](uint32_t k, uint32_t) {
      if (bin1(k) == b1) atomicAdd(&sm.row.hist[bin2(k)], 1u);
    });
    __syncthreads();
    uint32_t above2;
    hist_find<T>(sm.row.hist, (uint32_t)p.K - above, sm.row.sc, b2, above2);
  }
  // the band: the chosen bin's score range (from its edges, widened by 1 %
  // of a bin on each side, far more than the rounding of the bin
  // arithmetic; the top bin reaches the largest score), then E on each
  // side; the K-th largest lies in the bin
  double blo = (double)tau + ((double)b1 - 0.01) * (double)W;
  double bhi = b1 >= 4095u ? (double)order_key_f32(KX) : (double)tau + ((double)b1 + 1.01) * (double)W;
  if (two) {
    const double W2 = 1.0 / (double)iW2;
    if (b2 > 0u) blo = fmax(blo, (double)lo2 + ((double)b2 - 0.01) * W2);
    if (b2 < 4095u) bhi = fmin(bhi, (double)lo2 + ((double)b2 + 1.01) * W2);
  }
  const uint32_t klo = f32_order_key(nextafterf((float)(blo - (double)E), -INFINITY));
  const uint32_t khi = f32_order_key(nextafterf((float)(bhi + (double)E), INFINITY));
  if (klo < f32_order_key(tau)) return fallback();   // part of the band may lie below tau
  uint32_t n_in = 0u;
  each([&](uint32_t k, uint32_t j) {
    if (k > khi) {
      atomicOr(&sm.bm[j >> 5], 1u << (j & 31));
      ++n_in;
    } else if (k >= klo) {
      const uint32_t slot = atomicAdd(&sm.row.run[0], 1u);
      if (slot < (uint32_t)kBandCap) {
        sm.row.band_j[slot] = j;
        sm.row.band_k[slot] = k;
      }
    }
  });
  n_in = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl_u32(n_in), 63);
  if (lane == 0 && n_in) atomicAdd(&sm.row.run[1], n_in);
  __syncthreads();
  const uint32_t nb = sm.row.run[0], tot_in = sm.row.run[1];
  if (nb > (uint32_t)kBandCap) return fallback();
  const uint32_t R2 = (uint32_t)p.K - tot_in;      // 1 <= R2 <= nb
  if (nb == R2) {
    // every band member is needed: no exact keys
    for (uint32_t e = tid; e < nb; e += T) atomicOr(&sm.bm[sm.row.band_j[e] >> 5], 1u << (sm.row.band_j[e] & 31));
  } else {
    for (uint32_t e = tid >> 4; e < nb; e += T / 16) {   // a quarter-wave per band member
      const float key = group_exact_key<16>(c.ir, sm.row.band_j[e], sm.qs, sm.wsg);
      if ((lane & 15) == 0) sm.row.band_k[e] = f32_order_key(key);
    }
    __syncthreads();
    band_mark<T>(sm.row.band_k, sm.row.band_j, nb, R2, sm.bm);
  }
  __syncthreads();
  emit_bitmap<T, kMaxWords>(p, c, sm.row, sm.bm, nwords);
}

static constexpr int kFzCap = 512;   // = keys per indexer chunk: a chunk can never overflow

// Zero-fill of counters by a kernel (a memset node would not be safe under
// graph capture).
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* x, int n, uint32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = v;
}

// ---------------------------------------------------------------- fused, many rows (prefill)
// One selection group of four weighted-ReLU heads, contexts up to 65536.
// (1) fzr_pilot: a workgroup takes 8 consecutive rows (their 4 heads are the
//     32 slot rows of the 32x32x16 MFMA) and scores the sampled keys (runs of
//     64 every 2048) for all of them; per row, a
//     wave finds the R-th largest sampled key (R for about 1.25 K survivors in
//     proportion, plus a margin) by three 8-bit radix passes over a per-wave
//     histogram, and tau is the lower edge of its 24-bit bin; a row short
//     enough for its list keeps every key (tau = -inf).
// (2) the filtered indexer appends survivors (order key, position) to
//     per-row lists (kFzrCap per row).
// (3) fzr_final: one 256-thread workgroup per row: the list into LDS, then the
//     certified selection over it (radix select, band, exact band keys,
//     bitmap); rows it cannot settle (too few or too many survivors, a band
//     reaching below tau, a band key that needs the wide accumulator) are
//     flagged, and fzr_redo recomputes them from the inputs.
constexpr int kFzrRows = 8;        // pilot rows per workgroup (4 heads each)
constexpr int kFzrSamples = 2048;  // sampled keys per row (contexts up to 65536)
constexpr int kFzrCap = 5632;      // survivors kept per row
constexpr int kFzrCtx = 65536;
constexpr int kFzrThreads = 256;   // final kernel: four waves per row

__global__ __launch_bounds__(256) void fzr_pilot_kernel(TopkParams p, float* tau) {
  __shared__ uint32_t sk[kFzrRows][kFzrSamples];
  __shared__ uint32_t hist[4][256];
  const IndexerParams& x = p.ix;
  const int b = blockIdx.y, r0 = blockIdx.x * kFzrRows;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos0 = L - p.Nq + r0;                             // position of the first row
  const int rlast = min(p.Nq - 1, r0 + kFzrRows - 1);
  const int nmax = min(L - p.Nq + rlast + 1, kFzrCtx);        // keys seen by the last row
  const int nruns = nmax > 0 ? (nmax + kPilotStride - 1) / kPilotStride : 0;
  const int ntiles = 2 * nruns;
  const bool fp8 = x.k.dt == DT_FP8;
  // A operand: slot col = 4 (row) + head, dims 32 half + 8 s + v
  bf16x8 A[4];
  {
    const int rr = col >> 2, h = col & 3;
    if (r0 + rr < p.Nq) {
      const uint16_t* qp =
          (const uint16_t*)x.q.p + b * x.q.s[0] + (int64_t)(r0 + rr) * x.q.s[1] + h * x.q.s[2] + 32 * half;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) A[s4] = *(const bf16x8*)(qp + 8 * s4);
    } else {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) A[s4] = (bf16x8){};
    }
  }
  // lane (key col, half): accumulator v holds slot 8 (v / 4) + 4 half + v % 4,
  // i.e. row 2 (v / 4) + half, head v % 4
  float wv[4][4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = min(r0 + 2 * gi + half, p.Nq - 1);
      wv[gi][t] = x.w[b * x.ws_[0] + (int64_t)r * x.ws_[1] + t * x.ws_[2]];
    }
  for (int i = tid; i < kFzrRows * kFzrSamples; i += 256) sk[i / kFzrSamples][i % kFzrSamples] = 0u;
  __syncthreads();
  constexpr int TB = 4;
  for (int tb = wid; tb < ntiles; tb += 4 * TB) {
    u32x4 raw[TB][4];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int tt = tb + 4 * u;
      int j = (tt >> 1) * kPilotStride + 32 * (tt & 1) + col;
      j = j < nmax ? j : nmax - 1;
      if (tt < ntiles) {
        if (fp8) {
          const uint8_t* kp = (const uint8_t*)x.k.p + b * x.k.s[0] + (int64_t)j * x.k.s[1] + 32 * half;
          raw[u][0] = *(const u32x4*)kp;
          raw[u][1] = *(const u32x4*)(kp + 16);
        } else {
          const uint16_t* kp = (const uint16_t*)x.k.p + b * x.k.s[0] + (int64_t)j * x.k.s[1] + 32 * half;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) raw[u][q4] = *(const u32x4*)(kp + 8 * q4);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int tt = tb + 4 * u;
      if (tt >= ntiles) break;
      u32x4 Bw[4];
      if (fp8) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const uint32_t w0 = raw[u][s4 >> 1][2 * (s4 & 1)], w1 = raw[u][s4 >> 1][2 * (s4 & 1) + 1];
          Bw[s4][0] = fp8x2_to_bf16x2<false>(w0);
          Bw[s4][1] = fp8x2_to_bf16x2<true>(w0);
          Bw[s4][2] = fp8x2_to_bf16x2<false>(w1);
          Bw[s4][3] = fp8x2_to_bf16x2<true>(w1);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) Bw[s4] = raw[u][s4];
      }
      f32x16 acc = {};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s4], *(const bf16x8*)&Bw[s4], acc, 0, 0, 0);
      const int j = (tt >> 1) * kPilotStride + 32 * (tt & 1) + col;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        float sv = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) sv = fmaf(wv[gi][t], __int_as_float(max(__float_as_int(acc[4 * gi + t]), 0)), sv);
        const int rr = 2 * gi + half;
        if (j <= pos0 + rr) sk[rr][32 * tt + col] = f32_order_key(sv);
      }
    }
  }
  __syncthreads();
  // per row (wave w: rows 2w, 2w + 1): the R-th largest sampled key
  for (int rr = 2 * wid; rr < 2 * wid + 2; ++rr) {
    const int r = r0 + rr;
    if (r >= p.Nq) break;
    const int n = min(pos0 + rr + 1, kFzrCtx);
    if (n <= p.K) {
      if (lane == 0) tau[(int64_t)b * p.Nq + r] = INFINITY;
      continue;
    }
    if (n <= kFzrCap) {          // the whole row fits the list: keep every key
      if (lane == 0) tau[(int64_t)b * p.Nq + r] = -INFINITY;
      continue;
    }
    const int slots = 2 * 32 * ((n + kPilotStride - 1) / kPilotStride);
    uint32_t m = 0;
    for (int i = lane; i < slots; i += 64) m += sk[rr][i] != 0u;
    m = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl_u32(m), 63);
    const uint64_t want = ((uint64_t)5 * p.K * m + 4ull * n - 1) / (4ull * n) + 16;  // ~1.25 K survivors
    uint32_t need = (uint32_t)min((uint64_t)m, want);
    if (need == 0) {
      if (lane == 0) tau[(int64_t)b * p.Nq + r] = -INFINITY;
      continue;
    }
    uint32_t prefix = 0;
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = 24 - 8 * pass;
#pragma unroll
      for (int q = 0; q < 4; ++q) hist[wid][4 * lane + q] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < slots; i += 64) {
        const uint32_t v = sk[rr][i];
        if (v != 0u && (pass == 0 || (v >> (sh + 8)) == prefix)) atomicAdd(&hist[wid][(v >> sh) & 255u], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t hb[4], cnt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hb[q] = hist[wid][4 * lane + q];
        cnt += hb[q];
      }
      const uint32_t incl = wave_prefix_incl_u32(cnt);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      const uint32_t above = total - incl;                  // members in higher lanes' bins
      uint32_t digit = 0, ab = 0;
      const bool mine = above < need && need <= above + cnt;
      if (mine) {
        uint32_t acc = above;
        for (int q = 3; q >= 0; --q) {
          if (acc + hb[q] >= need) {
            digit = 4 * lane + q;
            ab = acc;
            break;
          }
          acc += hb[q];
        }
      }
      const uint64_t bm = ballot(mine);
      const int src = bm ? __builtin_ctzll(bm) : 0;
      digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, src);
      ab = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
      prefix = (prefix << 8) | digit;
      need -= ab;
      __builtin_amdgcn_wave_barrier();
    }
    if (lane == 0) tau[(int64_t)b * p.Nq + r] = order_key_f32(prefix << 8);
  }
}

struct FzrWs {
  float* tau;          // [rows]
  float* kmax;         // [B][nchunk]
  uint32_t* cnt;       // [rows]
  uint32_t* ck;        // [rows][kFzrCap] order keys
  uint32_t* cj;        // [rows][kFzrCap] positions
  uint32_t* redo;      // [rows]
  int nchunk;
};

// about 50 KB: three workgroups per CU
struct FzrSmem {
  RowSmemF row;        // radix histogram, then band lists and the selected-position bitmap
  float qs[4 * 64];
  float wsg[4];
  uint32_t ck[kFzrCap];
  uint16_t cj[kFzrCap];   // positions < kFzrCtx
  float red[2 * (kFzrThreads / 64)];
};
static_assert(kFzrCtx / 32 <= 2048, "the bitmap fits the row area");

__global__ __launch_bounds__(kFzrThreads) __attribute__((amdgpu_waves_per_eu(3))) void fzr_final_kernel(TopkParams p,
                                                                                           FzrWs w) {
  constexpr int T = kFzrThreads;
  constexpr int NW = T / 64;
  __shared__ FzrSmem sm;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  RowCtx c = row_ctx(p, row);
  if (c.n <= p.K) {
    write_all(p, c, T);
    if (tid == 0) w.redo[row] = 0u;
    return;
  }
  const uint32_t n_cand = w.cnt[row];
  const float tau = w.tau[row];
  const int L = min(p.ctx_len ? p.ctx_len[c.b] : p.ctx, p.ctx);
  const int nch_k = min(w.nchunk, (L + 511) / 512);
  float km = 0.f, coef = 0.f;
  for (int i = tid; i < nch_k; i += T) km = fmaxf(km, w.kmax[(int64_t)c.b * w.nchunk + i]);
  for (int e = tid; e < c.ir.H * c.ir.d; e += T) {
    const int hh = e / c.ir.d;
    const float qv = (float)load_f64(c.ir.q, c.ir.qt, hh * c.ir.qh_stride + e % c.ir.d);
    sm.qs[e] = qv;
    coef = fmaf(fabsf(c.ir.w[hh * c.ir.w_stride]), fabsf(qv), coef);
  }
  if (tid < c.ir.H) sm.wsg[tid] = c.ir.w[tid * c.ir.w_stride];
  const bool fits = n_cand >= (uint32_t)p.K && n_cand <= (uint32_t)kFzrCap;
  uint32_t kmx = 0;
  if (fits) {
    const uint32_t* gk = w.ck + (int64_t)row * kFzrCap;
    const uint32_t* gj = w.cj + (int64_t)row * kFzrCap;
    for (uint32_t i = tid; i < n_cand; i += T) {
      const uint32_t k = gk[i];
      sm.ck[i] = k;
      sm.cj[i] = (uint16_t)gj[i];
      kmx = max(kmx, k);
    }
  }
  km = wave_max_dpp(km);
  coef = wave_sum_dpp(coef);
  kmx = wave_max_u32_dpp(kmx);
  if (lane == 63) {
    sm.red[wid] = km;
    sm.red[NW + wid] = coef;
    sm.row.sc[wid] = kmx;
  }
  const int nwords = (c.n + 31) >> 5;
  __syncthreads();
  float KM = 0.f, CO = 0.f;
  uint32_t KX = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    KM = fmaxf(KM, sm.red[v]);
    CO += sm.red[NW + v];
    KX = max(KX, sm.row.sc[v]);
  }
  c.eps = eps_of(p.ix, CO, KM);
  __syncthreads();
  bool ok = fits;
  if (ok) {
    // the certification band around the K-th largest key must lie above tau:
    // a K-th key below tau + 2 E (rounded up) fails the row
    const float E = 2.0f * c.eps * 1.0001f + 1e-30f;
    const uint32_t base = f32_order_key(tau);
    const uint32_t tlo = f32_order_key(nextafterf(nextafterf(tau + 2.0f * E, INFINITY), INFINITY));
    ok = resolve_candidates<T, RowSmemF, 4, true>(p, c, sm.row, sm.ck, sm.cj, sm.row.bm, n_cand, (uint32_t)p.K, base,
                                                 max(KX, base), tlo, 0xFFFFFFFFu, sm.qs, sm.wsg, nwords);
  }
  if (ok) emit_bitmap<T, kFzrCtx / 32>(p, c, sm.row, sm.row.bm, nwords);
  if (tid == 0) w.redo[row] = ok ? 0u : 1u;
}

// Rows flagged by fzr_final: recomputed from the indexer inputs by the
// ordered single-pass routine (every score formed again by one thread). Every
// workgroup scans all flags in row order; the k-th flagged row goes to
// workgroup k mod gridDim.x, so flagged rows spread over the grid.
__global__ __launch_bounds__(kR2Threads) void fzr_redo_kernel(TopkParams p, const uint32_t* redo, int rows) {
  __shared__ RowSmem sm;
  __shared__ uint32_t list[kR2Threads];
  __shared__ uint32_t nlist;
  __shared__ float qs[4 * 64];
  __shared__ float wsg[4];
  uint32_t seen = 0;                       // flagged rows before this block of rows
  for (int r0 = 0; r0 < rows; r0 += kR2Threads) {
    if (threadIdx.x == 0) nlist = 0u;
    const int row = r0 + (int)threadIdx.x;
    const bool f = row < rows && redo[row] != 0u;
    uint32_t tot;
    const uint32_t k = seen + block_prefix<kR2Threads>(f, sm.sc, tot);
    if (f && k % gridDim.x == blockIdx.x) list[atomicAdd(&nlist, 1u)] = (uint32_t)row;
    seen += tot;
    __syncthreads();
    const uint32_t nl = nlist;
    for (uint32_t q = 0; q < nl; ++q) {
      RowCtx c = row_ctx(p, (int)list[q]);
      for (int e = threadIdx.x; e < c.ir.H * c.ir.d; e += kR2Threads)
        qs[e] = (float)load_f64(c.ir.q, c.ir.qt, (e / c.ir.d) * c.ir.qh_stride + e % c.ir.d);
      if ((int)threadIdx.x < c.ir.H) wsg[threadIdx.x] = c.ir.relu ? c.ir.w[threadIdx.x * c.ir.w_stride] : 1.f;
      __syncthreads();
      row_topk_single<kR2Threads>(p, c, sm, [&](int i) { return recompute_score_lds(c.ir, qs, wsg, i); });
      if (p.count && threadIdx.x == 0) p.count[((int64_t)c.b * p.G + c.g) * p.Nq + c.r] = p.K;
      __syncthreads();
    }
  }
}

static bool fused_rows_ok(const TopkParams& p) {
  return p.certified && index_filter_rows_ok(p.ix) && p.ctx <= kFzrCtx && p.G == 1;
}


static bool fused_few_ok(const TopkParams& p) {
  const int64_t nchunk = (p.ctx + 511) / 512;
  return index_filter_ok(p.ix) && p.ctx <= kDecCap / kDecRun * kDecStride &&
         (p.ctx + 31) / 32 <= kMaxWords && nchunk <= kTkThreads &&
         nchunk * p.G * p.Nq * kFzCap < ((int64_t)1 << 31);   // 32-bit candidate offsets per request
}

bool topk_fused_ok(const TopkParams& p) { return fused_few_ok(p) || fused_rows_ok(p); }

size_t topk_fused_ws_bytes(const TopkParams& p) {
  const int64_t rows = (int64_t)p.B * p.G * p.Nq;
  const int64_t nchunk = (p.ctx + 511) / 512;
  if (!fused_few_ok(p))    // per-row lists: keys and positions, counts, tau, chunk bounds, redo flags
    return (size_t)(rows * 2 * kFzrCap + rows * 3 + (int64_t)p.B * nchunk) * 4;
  return (size_t)(rows + (int64_t)p.B * nchunk + rows * nchunk * (1 + 2 * kFzCap)) * 4;
}

static hipError_t launch_topk_fused_rows(const TopkParams& p, hipStream_t st) {
  const int rows = p.B * p.G * p.Nq;
  FzrWs w;
  w.nchunk = (p.ctx + 511) / 512;
  w.ck = (uint32_t*)p.ws;
  w.cj = w.ck + (int64_t)rows * kFzrCap;
  w.cnt = w.cj + (int64_t)rows * kFzrCap;
  w.redo = w.cnt + rows;
  w.tau = (float*)(w.redo + rows);
  w.kmax = w.tau + rows;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, w.cnt, rows, 0u);
  hipLaunchKernelGGL(fzr_pilot_kernel, dim3((p.Nq + kFzrRows - 1) / kFzrRows, p.B), dim3(256), 0, st, p, w.tau);
  IndexerParams ix = p.ix;
  ix.kmax = w.kmax;
  ix.tau = w.tau;
  ix.cand = w.ck;
  ix.cand_j = w.cj;
  ix.cand_n = w.cnt;
  ix.cap = kFzrCap;
  ix.err = nullptr;
  hipError_t e = launch_index_filter(ix, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fzr_final_kernel, dim3(rows), dim3(kFzrThreads), 0, st, p, w);
  hipLaunchKernelGGL(fzr_redo_kernel, dim3(min((rows + kR2Threads - 1) / kR2Threads, kRedoGrid)), dim3(kR2Threads),
                     0, st, p, w.redo, rows);
  return hipGetLastError();
}

hipError_t launch_topk_fused(const TopkParams& p, hipStream_t st) {
  if (!fused_few_ok(p)) return launch_topk_fused_rows(p, st);
  const int rows = p.B * p.G * p.Nq;
  FzWs w;
  w.nchunk = (p.ctx + 511) / 512;
  w.cap = kFzCap;
  w.cand = (u32x2*)p.ws;                                  // first: 8-byte aligned
  w.tau = (float*)(w.cand + (int64_t)rows * w.nchunk * w.cap);
  w.kmax = w.tau + rows;
  w.cand_n = (uint32_t*)(w.kmax + (int64_t)p.B * w.nchunk);
  hipLaunchKernelGGL(fz_pilot_kernel, dim3(rows), dim3(kTkThreads), 0, st, p, w.tau);
  IndexerParams ix = p.ix;
  ix.kmax = w.kmax;
  ix.tau = w.tau;
  ix.cand = (uint32_t*)w.cand;
  ix.cand_n = w.cand_n;
  ix.cap = w.cap;
  ix.err = nullptr;
  hipError_t e = launch_index_filter(ix, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fz_final_kernel, dim3(rows), dim3(kTkThreads), 0, st, p, w);
  return hipGetLastError();
}

static bool use_multi(const TopkParams& p) {
  const int64_t rows = (int64_t)p.B * p.G * p.Nq;
  return rows <= 1024 && p.ctx >= 4 * kMtChunk && (p.ctx + 31) / 32 <= kMaxWords &&
         (p.ctx + kMtChunk - 1) / kMtChunk <= 64;
}

size_t topk_ws_bytes(const TopkParams& p) {
  if (!use_multi(p)) return p.ctx <= 32 * kR2Words ? (size_t)p.B * p.G * p.Nq * sizeof(uint32_t) : 0;   // redo flags
  const int64_t rows = (int64_t)p.B * p.G * p.Nq;
  const int64_t words = (p.ctx + 31) / 32;
  const int64_t nchunk = (p.ctx + kMtChunk - 1) / kMtChunk;
  return (size_t)rows * (4096 + nchunk * 2 + 1 + words + 2 * nchunk * kChunkCand) * sizeof(uint32_t);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const int rows = p.B * p.G * p.Nq;
  if (!use_multi(p)) {
    if (p.ctx <= 32 * kR2Words) {
      uint32_t* redo = (uint32_t*)p.ws;
      hipLaunchKernelGGL(topk_row2_kernel, dim3(rows), dim3(kR2Threads), 0, st, p, redo);
      hipLaunchKernelGGL(topk_redo_kernel, dim3(min((rows + kR2Threads - 1) / kR2Threads, kRedoGrid)), dim3(kR2Threads),
                         0, st, p, redo, rows);
    } else
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
