// Workgroup-level selection primitives: ordered compaction and radix select.
//
// Keys are order-preserving 32-bit images of float32 values (f32_order_key),
// so "largest float" is "largest key". Radix select finds the R-th largest
// key of a set in three histogram passes (12 + 12 + 8 bits) over LDS, using
// ballots and wave prefix counts for the bin search. Selections break ties
// by index (lower first) through an ordered pass with a running tie rank.
#pragma once
#include "common.h"

namespace sp {

// Exclusive prefix count of `flag` over the workgroup in thread order, and
// the total. `scratch` holds >= 1 + waves uint32 in LDS. Two barriers.
template <int T>
SP_DEV uint32_t block_prefix(bool flag, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = T / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t m = ballot(flag);
  const uint32_t below = lanes_below(m);
  if (lane == 0) scratch[wid] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = scratch[w];
    base += (w < wid) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + below;
}

// Exclusive prefix sum of `v` over the workgroup in thread order, and the total.
template <int T>
SP_DEV uint32_t block_scan_sum(uint32_t v, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = T / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t incl = wave_prefix_incl_u32(v);
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = scratch[w];
    base += (w < wid) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Find the R-th largest key (R >= 1, R <= number of included elements).
// get(i, key) returns true when element i takes part. Keys are taken relative
// to `base` and must lie in [base, base + 2^bits) for included elements; the
// bits are consumed from the top in digits of at most 12. On return: t = that
// key (absolute), above = number of included elements with key > t.
// With thi given, the passes may stop early, once the keys left in the chosen
// bin span at most tol as floats (order keys of finite floats): then t and
// *thi are the ends of that bin (the R-th largest lies in [t, *thi]) and
// above counts the elements above the bin; otherwise *thi = t.
template <int T, typename Get>
SP_DEV void radix_select(int n, uint32_t R, Get get, uint32_t* hist, uint32_t* sc,
                         uint32_t& t, uint32_t& above, uint32_t base = 0u, int bits = 32,
                         uint32_t* thi = nullptr, float tol = -1.f) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int NW = T / 64;
  uint32_t prefix = 0, pmask = 0, acc_above = 0, need = R;
  int left = bits;
#pragma unroll 1
  while (left > 0) {
    const int width = left >= 12 ? 12 : left;
    const int sh = left - width;
    const int nb = 1 << width;
    const uint32_t dmask = (uint32_t)(nb - 1);
    for (int i = tid; i < nb; i += T) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += T) {
      uint32_t k;
      if (get(i, k)) {
        k -= base;
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> sh) & dmask], 1u);
      }
    }
    __syncthreads();
    // thread owns bins [lo, lo+per); suffix sums from the top
    const int per = nb >= T ? nb / T : 1;
    const int lo = tid * per;
    uint32_t mine = 0;
    if (lo < nb)
      for (int q = 0; q < per; ++q) mine += hist[lo + q];
    // inclusive suffix sum within the wave (higher lanes own higher bins)
    const uint32_t pin = wave_prefix_incl_u32(mine);
    const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)pin, 63) - pin + mine;
    if (lane == 0) sc[wid] = v;   // wave total
    __syncthreads();
    uint32_t higher_waves = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) higher_waves += (w > wid) ? sc[w] : 0u;
    uint32_t cum = higher_waves + (v - mine);   // elements in bins above mine
    if (lo < nb && cum < need && cum + mine >= need) {
      for (int q = per - 1; q >= 0; --q) {
        const uint32_t h = hist[lo + q];
        if (cum + h >= need) {
          sc[NW] = (uint32_t)(lo + q);
          sc[NW + 1] = cum;
          break;
        }
        cum += h;
      }
    }
    __syncthreads();
    const uint32_t bin = sc[NW], ab = sc[NW + 1];
    __syncthreads();
    acc_above += ab;
    need -= ab;
    prefix |= bin << sh;
    pmask |= dmask << sh;
    left = sh;
    if (thi && left > 0) {
      const float flo = order_key_f32(base + prefix);
      const float fhi = order_key_f32(base + (prefix | ((1u << left) - 1u)));
      if (fhi - flo <= tol) break;          // false for a non-finite end: keep refining
    }
  }
  t = prefix + base;
  if (thi) *thi = base + (prefix | (left > 0 ? (1u << left) - 1u : 0u));
  above = acc_above;
}

}  // namespace sp
