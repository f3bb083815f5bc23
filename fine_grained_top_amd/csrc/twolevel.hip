// Two-level selection ("Sparse Attention Is Reshaping Production AI",
// per-token routing: a coarse block pass finds candidate regions cheaply, a
// fine pass picks the top-K tokens inside them).
//
//  * tl_pool: each complete block's indexer key is the mean of its tokens'
//    indexer keys, summed in float64 and rounded once to float32 (a per-block
//    cache that a decode loop extends one block at a time).
//  * two_level (one 512-thread workgroup per row): the indexer's score of
//    the row's query heads on every complete past block key picks the
//    top_blocks blocks; the candidates are their tokens plus the tokens of
//    the query's own incomplete block; the indexer's score of each candidate
//    picks the K best. Both picks are certified like the token top-K: float32
//    scores with a rigorous error bound, the band around the threshold
//    rescored exactly (a quarter-wave per key), ties to the lower index.
#include "common.h"
#include "exact.h"
#include "internal.h"
#include "rowselect.h"

namespace sp {

constexpr int kTlThreads = 512;
constexpr int kTlBandCap = 2048;

struct TlSmem {
  uint32_t keys[kTlMaxCand];     // order keys: blocks (first pick), then candidate tokens
  int32_t cpos[kTlMaxCand];      // candidate positions, ascending
  uint32_t hist[4096];
  uint32_t band_j[kTlBandCap];
  uint32_t band_k[kTlBandCap];
  uint32_t bm[kTlMaxCand / 32];  // selection bitmap of the current pick
  float qs[4096];                // the group's query heads [hpg][d_I] as float
  float wsg[64];                 // their weights (1 in DOT mode)
  uint32_t sc[16];
  uint32_t run[4];
  float red[32];
};

SP_DEV float key_elem(const void* k, int kt, int64_t i) {
  if (kt == DT_F32) return ((const float*)k)[i];
  if (kt == DT_BF16) return bf16_to_f32(((const uint16_t*)k)[i]);
  return fp8_to_f32(((const uint8_t*)k)[i]);
}

// float32 score of one key row (any summation order is covered by the bound)
// and the row's largest |k| element. With d = 64 the row is loaded by 16-byte
// vector loads, all issued before the first use (rows are 16-byte aligned).
SP_DEV float tl_score(const TlSmem& sm, const IndexerRow& ir, int64_t j, float& kabs) {
  const int64_t ko = j * ir.k_stride;
  if (ir.d == 64) {
    float kv[64];
    if (ir.kt == DT_F32) {
      const f32x4* kp = (const f32x4*)((const float*)ir.k + ko);
      f32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = kp[i];
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[4 * i + e] = v[i][e];
    } else if (ir.kt == DT_BF16) {
      const u32x4* kp = (const u32x4*)((const uint16_t*)ir.k + ko);
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = kp[i];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[8 * i + 2 * e] = bf16_to_f32(v[i][e] & 0xFFFFu);
          kv[8 * i + 2 * e + 1] = bf16_to_f32(v[i][e] >> 16);
        }
    } else {
      const u32x4* kp = (const u32x4*)((const uint8_t*)ir.k + ko);
      u32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = kp[i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[i][e], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[i][e], true);
          kv[16 * i + 4 * e + 0] = lo[0];
          kv[16 * i + 4 * e + 1] = lo[1];
          kv[16 * i + 4 * e + 2] = hi[0];
          kv[16 * i + 4 * e + 3] = hi[1];
        }
    }
#pragma unroll
    for (int c = 0; c < 64; ++c) kabs = fmaxf(kabs, fabsf(kv[c]));
    float s = 0.f;
    for (int h = 0; h < ir.H; ++h) {
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < 64; ++c) d = fmaf(sm.qs[h * 64 + c], kv[c], d);
      s = ir.relu ? fmaf(sm.wsg[h], fmaxf(d, 0.f), s) : d;
    }
    return s;
  }
  float s = 0.f;
  for (int h = 0; h < ir.H; ++h) {
    float d = 0.f;
    for (int c = 0; c < ir.d; ++c) {
      const float kv = key_elem(ir.k, ir.kt, ko + c);
      if (h == 0) kabs = fmaxf(kabs, fabsf(kv));
      d = fmaf(sm.qs[h * ir.d + c], kv, d);
    }
    s = ir.relu ? fmaf(sm.wsg[h], fmaxf(d, 0.f), s) : d;
  }
  return s;
}

// Certified top-R of keys[0..n) (R < n <= kTlMaxCand; keys within eps of the
// exact keys, eps < 0: the keys are exact) into bm, ties to the lower index.
// ex16(i): exact key of candidate i by a 16-lane group; ex1(i): by one thread.
template <int T, typename Ex16, typename Ex1>
SP_DEV void certified_pick(TlSmem& sm, int n, uint32_t R, float eps, Ex16 ex16, Ex1 ex1) {
  const int tid = threadIdx.x, lane = tid & 63;
  static_assert(kTlMaxCand / 32 <= T && kTlMaxCand / 32 <= 256, "one bitmap word per thread");
  uint32_t t, above;
  radix_select<T>(n, R, [&](int i, uint32_t& k) { k = sm.keys[i]; return true; }, sm.hist, sm.sc, t, above);
  uint32_t klo = t, khi = t;
  const bool certified = eps >= 0.f;
  if (certified) {
    const float tf = order_key_f32(t);
    const float E = 2.0f * eps * 1.0001f + 1e-30f;
    klo = f32_order_key(nextafterf(tf - E, -INFINITY));
    khi = f32_order_key(nextafterf(tf + E, INFINITY));
  }
  // bits of the keys above the band (hist[w]) and in it (hist[256 + w])
  const int nwords = (n + 31) >> 5;
  for (int c = tid >> 6; 64 * c < n; c += T / 64) {
    const int i = 64 * c + lane;
    const uint32_t k = i < n ? sm.keys[i] : 0u;
    const uint64_t min_ = ballot(i < n && k > khi);
    const uint64_t mbd = ballot(i < n && k >= klo && k <= khi);
    if (lane == 0) {
      sm.hist[2 * c] = (uint32_t)min_;
      sm.hist[256 + 2 * c] = (uint32_t)mbd;
    } else if (lane == 1 && 2 * c + 1 < nwords) {
      sm.hist[2 * c + 1] = (uint32_t)(min_ >> 32);
      sm.hist[256 + 2 * c + 1] = (uint32_t)(mbd >> 32);
    }
  }
  __syncthreads();
  const uint32_t win = tid < nwords ? sm.hist[tid] : 0u;
  const uint32_t wbd = tid < nwords ? sm.hist[256 + tid] : 0u;
  uint32_t tot;
  const uint32_t pre = block_scan_sum<T>(((uint32_t)__popc(wbd) << 16) | (uint32_t)__popc(win), sm.sc, tot);
  const uint32_t n_in = tot & 0xFFFFu, n_band = tot >> 16;
  const uint32_t R2 = R - n_in;                  // >= 1
  const bool cached = n_band <= (uint32_t)kTlBandCap;
  if (cached) {
    uint32_t slot = pre >> 16;
    for (uint32_t m = wbd; m; m &= m - 1, ++slot) {
      const int i = 32 * tid + __ffs(m) - 1;
      sm.band_j[slot] = (uint32_t)i;
      sm.band_k[slot] = sm.keys[i];
    }
  }
  if (tid < kTlMaxCand / 32) sm.bm[tid] = tid < nwords ? win : 0u;
  __syncthreads();

  if (!cached) {
    // rare: exact keys of the band recomputed by each thread in ordered passes
    uint32_t t2, above2;
    radix_select<T>(n, R2,
                    [&](int i, uint32_t& k) {
                      const uint32_t ck = sm.keys[i];
                      if (ck < klo || ck > khi) return false;
                      k = certified ? f32_order_key(ex1(i)) : ck;
                      return true;
                    },
                    sm.hist, sm.sc, t2, above2);
    const uint32_t need_eq = R2 - above2;
    uint32_t run_eq = 0;
    for (int base = 0; base < n; base += T) {
      const int i = base + tid;
      bool sel = false, eq = false;
      if (i < n) {
        const uint32_t ck = sm.keys[i];
        if (ck >= klo && ck <= khi) {
          const uint32_t ex = certified ? f32_order_key(ex1(i)) : ck;
          eq = ex == t2;
          sel = ex > t2;
        }
      }
      uint32_t neq;
      const uint32_t er = run_eq + block_prefix<T>(eq, sm.sc, neq);
      run_eq += neq;
      if (sel || (eq && er < need_eq)) atomicOr(&sm.bm[i >> 5], 1u << (i & 31));
    }
    __syncthreads();
    return;
  }
  if (certified) {
    for (uint32_t e = tid >> 4; e < n_band; e += T / 16) {
      const float key = ex16(sm.band_j[e]);
      if ((lane & 15) == 0) sm.band_k[e] = f32_order_key(key);
    }
    __syncthreads();
  }
  uint32_t t2, above2;
  radix_select<T>((int)n_band, R2, [&](int i, uint32_t& k) { k = sm.band_k[i]; return true; }, sm.hist, sm.sc, t2,
                  above2);
  const uint32_t need_eq = R2 - above2;
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
      atomicOr(&sm.bm[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
}

// Block means of the indexer keys: one workgroup per (block, key head, request).
__global__ __launch_bounds__(256) void tl_pool_kernel(TwoLevelParams q) {
  const IndexerParams& x = q.t.ix;
  const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = min(q.t.ctx_len ? q.t.ctx_len[b] : x.ctx, x.ctx);
  const int bs = 1 << q.lgbs;
  if (blk >= (L >> q.lgbs)) return;
  for (int c = threadIdx.x; c < x.d_I; c += blockDim.x) {
    double s = 0.0;
    const int64_t base = b * x.k.s[0] + (int64_t)blk * bs * x.k.s[1] + g * x.k.s[2] + c;
    for (int t = 0; t < bs; ++t) s += (double)key_elem(x.k.p, x.k.dt, base + t * x.k.s[1]);
    q.kp[b * q.kps[0] + blk * q.kps[1] + g * q.kps[2] + c] = (float)(s / (double)bs);
  }
}

__global__ __launch_bounds__(kTlThreads) void two_level_kernel(TwoLevelParams q) {
  constexpr int T = kTlThreads;
  __shared__ TlSmem sm;
  const TopkParams& p = q.t;
  const IndexerParams& x = p.ix;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int r = row % p.Nq, g = (row / p.Nq) % p.G, b = row / (p.Nq * p.G);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  int32_t* out = p.idx + b * p.is[0] + g * p.is[1] + r * p.is[2];
  int32_t* cnt = p.count ? p.count + ((int64_t)b * p.G + g) * p.Nq + r : nullptr;
  const int K = q.blocks_only ? q.nb : p.K;
  if (pos < 0) {
    for (int i = tid; i < K; i += T) out[i] = -1;
    if (cnt && tid == 0) *cnt = 0;
    return;
  }
  const int bs = 1 << q.lgbs;
  const int nbe = (pos + 1) >> q.lgbs;             // complete past blocks
  const int nopen = pos + 1 - (nbe << q.lgbs);     // tokens of the open block

  // the group's query heads and weights as float (exact copies)
  const IndexerRow irt = indexer_row(x, b, g, r);
  IndexerRow irp = irt;                            // the same row on the block keys
  const int kg = x.G_k == 1 ? 0 : g;
  irp.k = q.kp + b * q.kps[0] + kg * q.kps[2];
  irp.kt = DT_F32;
  irp.k_stride = q.kps[1];
  for (int i = tid; i < irt.H * irt.d; i += T) {
    const int h = i / irt.d, c = i % irt.d;
    sm.qs[i] = (float)load_f64(irt.q, irt.qt, h * irt.qh_stride + c);
  }
  if (tid < irt.H) sm.wsg[tid] = irt.relu ? irt.w[tid * irt.w_stride] : 1.f;
  __syncthreads();
  // CO of the bound: sum over heads and dims of |w_h q_hc|
  float co = 0.f;
  for (int i = tid; i < irt.H * irt.d; i += T) co = fmaf(fabsf(sm.wsg[i / irt.d]), fabsf(sm.qs[i]), co);

  // ---- first pick: blocks
  if (nbe > q.nb) {
    float kabs = 0.f;
    for (int blk = tid; blk < nbe; blk += T) sm.keys[blk] = f32_order_key(tl_score(sm, irp, blk, kabs));
    float km = wave_max(kabs), cs = wave_sum(co);
    if ((tid & 63) == 0) {
      sm.red[tid >> 6] = km;
      sm.red[16 + (tid >> 6)] = cs;
    }
    __syncthreads();
    float KM = 0.f, CO = 0.f;
    for (int w = 0; w < T / 64; ++w) {
      KM = fmaxf(KM, sm.red[w]);
      CO += sm.red[16 + w];
    }
    __syncthreads();
    certified_pick<T>(sm, nbe, (uint32_t)q.nb, eps_of(x, CO, KM),
                      [&](int i) { return group_exact_key<16>(irp, i, sm.qs, sm.wsg); },
                      [&](int i) { return exact_key(irp, i); });
  } else {
    for (int w = tid; w < kTlMaxCand / 32; w += T) {
      const int lo = 32 * w;
      sm.bm[w] = lo >= nbe ? 0u : (nbe - lo >= 32 ? 0xFFFFFFFFu : (1u << (nbe - lo)) - 1u);
    }
    __syncthreads();
  }

  if (q.blocks_only) {                             // the chosen blocks, ascending
    const int nwb = (nbe + 31) >> 5;
    const uint32_t wv = tid < nwb ? sm.bm[tid] : 0u;
    uint32_t nsel;
    uint32_t opos = block_scan_sum<T>((uint32_t)__popc(wv), sm.sc, nsel);
    for (uint32_t m = wv; m; m &= m - 1, ++opos)
      if (opos < (uint32_t)K) out[opos] = 32 * tid + __ffs(m) - 1;
    for (int i = (int)nsel + tid; i < K; i += T) out[i] = -1;
    if (cnt && tid == 0) *cnt = min((int)nsel, K);
    return;
  }

  // ---- candidates: the chosen blocks' tokens, ascending, then the open block
  {
    const int nwb = (nbe + 31) >> 5;
    const uint32_t wv = tid < nwb ? sm.bm[tid] : 0u;
    uint32_t tot;
    uint32_t at = block_scan_sum<T>((uint32_t)__popc(wv) << q.lgbs, sm.sc, tot);
    for (uint32_t m = wv; m; m &= m - 1) {
      const int blk = 32 * tid + __ffs(m) - 1;
      for (int t2 = 0; t2 < bs; ++t2) sm.cpos[at + t2] = (blk << q.lgbs) + t2;
      at += bs;
    }
    for (int i = tid; i < nopen; i += T) sm.cpos[tot + i] = (nbe << q.lgbs) + i;
    if (tid == 0) sm.run[3] = tot + nopen;
    __syncthreads();
  }
  const int nc = (int)sm.run[3];

  // ---- second pick: tokens
  if (nc <= K) {
    for (int i = tid; i < K; i += T) out[i] = i < nc ? sm.cpos[i] : -1;
    if (cnt && tid == 0) *cnt = nc;
    return;
  }
  {
    float kabs = 0.f;
    for (int i = tid; i < nc; i += T) sm.keys[i] = f32_order_key(tl_score(sm, irt, sm.cpos[i], kabs));
    float km = wave_max(kabs), cs = wave_sum(co);
    if ((tid & 63) == 0) {
      sm.red[tid >> 6] = km;
      sm.red[16 + (tid >> 6)] = cs;
    }
    __syncthreads();
    float KM = 0.f, CO = 0.f;
    for (int w = 0; w < T / 64; ++w) {
      KM = fmaxf(KM, sm.red[w]);
      CO += sm.red[16 + w];
    }
    __syncthreads();
    certified_pick<T>(sm, nc, (uint32_t)K, eps_of(x, CO, KM),
                      [&](int i) { return group_exact_key<16>(irt, sm.cpos[i], sm.qs, sm.wsg); },
                      [&](int i) { return exact_key(irt, sm.cpos[i]); });
  }
  // ---- the chosen candidates, ascending
  const int nw = (nc + 31) >> 5;
  const uint32_t wsel = tid < nw ? sm.bm[tid] : 0u;
  uint32_t nsel;
  uint32_t opos = block_scan_sum<T>((uint32_t)__popc(wsel), sm.sc, nsel);
  for (uint32_t m = wsel; m; m &= m - 1, ++opos)
    if (opos < (uint32_t)K) out[opos] = sm.cpos[32 * tid + __ffs(m) - 1];
  if (cnt && tid == 0) *cnt = K;
}

// ---------------------------------------------------------------- blocks only, one wave per row
// The coarse pick alone for many rows (prefill): one wave per row, four rows
// of one (request, group) per workgroup, which share every 64-block chunk of
// the block-key cache staged in LDS (lane l scores block 64 c + l of chunk c,
// so each lane holds the keys of blocks l, 64 + l, ..., 448 + l). The
// R-th largest computed key t comes from removing the wave's maximum value
// (all its copies) until R keys are out; keys above t + 2 eps are in the
// exact selection, keys below t - 2 eps are out, and only when the band
// between holds more keys than the free slots are its members rescored
// exactly and ranked by (exact key desc, block asc).
constexpr int kGbRows = 4;           // rows (waves) per workgroup
constexpr int kGbSlots = 8;          // blocks per lane: up to 512 blocks per request
constexpr int kGbStride = 65;        // LDS row stride of a staged block key (floats)

__global__ __launch_bounds__(64 * kGbRows) void group_block_pick_kernel(TwoLevelParams q) {
  __shared__ float kb[64 * kGbStride];
  __shared__ float qsw[kGbRows][4 * 64];
  const TopkParams& p = q.t;
  const IndexerParams& x = p.ix;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = blockIdx.y, b = blockIdx.z;
  const int r = blockIdx.x * kGbRows + wid;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int rlast = min(blockIdx.x * kGbRows + kGbRows - 1, p.Nq - 1);
  const int nbe_max = max(0, L - p.Nq + rlast + 1) >> q.lgbs;   // blocks any row of this workgroup sees
  const bool live = r < p.Nq;
  const int pos = L - p.Nq + r;
  const int nbe = live && pos >= 0 ? (pos + 1) >> q.lgbs : 0;
  const int R = q.nb;
  const int kg = x.G_k == 1 ? 0 : g;
  IndexerRow ir{};
  float co = 0.f;
  if (live) {
    ir = indexer_row(x, b, g, r);
    for (int e = lane; e < ir.H * 64; e += 64) {
      const int h = e >> 6;
      const float qv = (float)load_f64(ir.q, ir.qt, h * ir.qh_stride + (e & 63));
      qsw[wid][e] = qv;
      co = fmaf(ir.relu ? fabsf(ir.w[h * ir.w_stride]) : 1.f, fabsf(qv), co);
    }
  }
  float wsg[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wsg[h] = live && h < ir.H ? (ir.relu ? ir.w[h * ir.w_stride] : 1.f) : 0.f;
  const float* kbase = q.kp + b * q.kps[0] + kg * q.kps[2];
  uint32_t key[kGbSlots];
  float kabs = 0.f;
#pragma unroll
  for (int c = 0; c < kGbSlots; ++c) {
    key[c] = 0u;
    if (64 * c >= nbe_max) continue;                // uniform over the workgroup
    __syncthreads();                                // the previous chunk is consumed
    for (int e = tid; e < 64 * 16; e += 64 * kGbRows) {
      const int bl = e >> 4, c4 = (e & 15) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (64 * c + bl < nbe_max) v = *(const float4*)(kbase + (int64_t)(64 * c + bl) * q.kps[1] + c4);
      float* d = kb + bl * kGbStride + c4;
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
    __syncthreads();
    const int blk = 64 * c + lane;
    if (live && blk < nbe) {
      const float* kr = kb + lane * kGbStride;
      float dd[4] = {0.f, 0.f, 0.f, 0.f};
      for (int e = 0; e < 64; ++e) {
        const float kv = kr[e];
        kabs = fmaxf(kabs, fabsf(kv));
#pragma unroll
        for (int h = 0; h < 4; ++h)
          if (h < ir.H) dd[h] = fmaf(qsw[wid][h * 64 + e], kv, dd[h]);
      }
      float sc = 0.f;
      if (ir.relu) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          if (h < ir.H) sc = fmaf(wsg[h], fmaxf(dd[h], 0.f), sc);
      } else {
        sc = dd[0];
      }
      key[c] = f32_order_key(sc);                   // > 0 for every finite score
    }
  }
  if (!live) return;                                // no barrier below
  int32_t* out = p.idx + b * p.is[0] + g * p.is[1] + r * p.is[2];
  int32_t* cnt = p.count ? p.count + ((int64_t)b * p.G + g) * p.Nq + r : nullptr;
  if (nbe <= R) {                                   // every complete block (none when pos < 0)
    for (int i = lane; i < R; i += 64) out[i] = i < nbe ? i : -1;
    if (cnt && lane == 0) *cnt = nbe;
    return;
  }
  // the R-th largest computed key
  uint32_t wk[kGbSlots];
#pragma unroll
  for (int c = 0; c < kGbSlots; ++c) wk[c] = key[c];
  uint32_t removed = 0, t = 0;
  while (true) {
    uint32_t m = 0u;
#pragma unroll
    for (int c = 0; c < kGbSlots; ++c) m = max(m, wk[c]);
    m = wave_max_u32_dpp(m);
    uint32_t n = 0;
#pragma unroll
    for (int c = 0; c < kGbSlots; ++c) n += (uint32_t)__popcll(ballot(wk[c] == m));
    if (removed + n >= (uint32_t)R || m == 0u) {
      t = m;
      break;
    }
    removed += n;
#pragma unroll
    for (int c = 0; c < kGbSlots; ++c)
      if (wk[c] == m) wk[c] = 0u;
  }
  // certified band around t
  const float KM = wave_max_dpp(kabs);
  const float CO = wave_sum_dpp(co);
  const float E = 2.0f * eps_of(x, CO, KM) * 1.0001f + 1e-30f;
  const float tf = order_key_f32(t);
  const uint32_t klo = f32_order_key(nextafterf(tf - E, -INFINITY));
  const uint32_t khi = f32_order_key(nextafterf(tf + E, INFINITY));
  bool chosen[kGbSlots], band[kGbSlots];
  uint32_t n_in = 0, n_band = 0;
#pragma unroll
  for (int c = 0; c < kGbSlots; ++c) {
    chosen[c] = key[c] > khi;
    band[c] = key[c] != 0u && key[c] >= klo && key[c] <= khi;
    n_in += (uint32_t)__popcll(ballot(chosen[c]));
    n_band += (uint32_t)__popcll(ballot(band[c]));
  }
  const uint32_t R2 = (uint32_t)R - n_in;           // n_in + n_band >= R (every key >= t is in or in the band)
  if (n_band <= R2) {
#pragma unroll
    for (int c = 0; c < kGbSlots; ++c) chosen[c] = chosen[c] || band[c];
  } else {
    // exact keys of the band, ranked by (exact key desc, block asc)
    IndexerRow irp = ir;
    irp.k = kbase;
    irp.kt = DT_F32;
    irp.k_stride = q.kps[1];
    uint32_t ex[kGbSlots];
#pragma unroll
    for (int c = 0; c < kGbSlots; ++c) ex[c] = band[c] ? f32_order_key(exact_key(irp, 64 * c + lane)) : 0u;
    for (uint32_t k = 0; k < R2; ++k) {
      uint32_t m = 0u;
#pragma unroll
      for (int c = 0; c < kGbSlots; ++c) m = max(m, ex[c]);
      m = wave_max_u32_dpp(m);
      uint32_t inv = 0u;                             // the lowest block holding m, as 0xFFFFFFFF - block
#pragma unroll
      for (int c = 0; c < kGbSlots; ++c)
        if (m != 0u && ex[c] == m) inv = max(inv, 0xFFFFFFFFu - (uint32_t)(64 * c + lane));
      const uint32_t win = 0xFFFFFFFFu - wave_max_u32_dpp(inv);
#pragma unroll
      for (int c = 0; c < kGbSlots; ++c)
        if ((uint32_t)(64 * c + lane) == win) {
          chosen[c] = true;
          ex[c] = 0u;
        }
    }
  }
  uint32_t base = 0;
#pragma unroll
  for (int c = 0; c < kGbSlots; ++c) {
    const uint64_t m = ballot(chosen[c]);
    if (chosen[c]) out[base + lanes_below(m)] = 64 * c + lane;
    base += (uint32_t)__popcll(m);
  }
  if (cnt && lane == 0) *cnt = R;
}

static bool group_block_pick_ok(const TwoLevelParams& q) {
  const IndexerParams& x = q.t.ix;
  return q.blocks_only && x.d_I == 64 && x.hpg <= 4 && (x.ctx >> q.lgbs) <= 64 * kGbSlots && q.nb <= 64;
}

hipError_t launch_pool_index_keys(const TwoLevelParams& q, hipStream_t st) {
  const IndexerParams& x = q.t.ix;
  const int nblk = x.ctx >> q.lgbs;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(tl_pool_kernel, dim3(nblk, x.G_k, x.B), dim3(64), 0, st, q);
  return hipGetLastError();
}

hipError_t launch_two_level(const TwoLevelParams& q, hipStream_t st) {
  if (group_block_pick_ok(q)) {
    hipLaunchKernelGGL(group_block_pick_kernel, dim3((q.t.Nq + kGbRows - 1) / kGbRows, q.t.G, q.t.B),
                       dim3(64 * kGbRows), 0, st, q);
    return hipGetLastError();
  }
  const int rows = q.t.B * q.t.G * q.t.Nq;
  hipLaunchKernelGGL(two_level_kernel, dim3(rows), dim3(kTlThreads), 0, st, q);
  return hipGetLastError();
}

}  // namespace sp
