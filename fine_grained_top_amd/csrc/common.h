// Device helpers shared by the libspattn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SP_DEV __device__ __forceinline__

namespace sp {

constexpr int kWave = 64;

// Workgroup id -> work item such that each of the 8 XCDs (workgroups go to
// them round-robin by id) takes a contiguous range of items, so that
// neighbouring items, which read the same data, meet in one XCD's L2. The
// grid holds 8 * per workgroups, per = ceil(items / 8); ids that map past
// the last item have nothing to do.
SP_DEV int xcd_item(int wg, int per) { return (wg & 7) * per + (wg >> 3); }

SP_DEV float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
SP_DEV uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

// Two fp8 E4M3FN codes (bytes 2*HI, 2*HI+1 of w) -> packed bf16 pair, exact
// (every E4M3FN value, subnormals included, is a bf16 value): one gfx950
// scaled conversion with unit scale.
template <bool HI>
SP_DEV uint32_t fp8x2_to_bf16x2(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

SP_DEV float fp8_to_f32(uint32_t code) {
  auto f = __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFFu, false);
  return f[0];
}

// Order-preserving map float -> uint32 (larger float => larger key); -0 -> +0.
SP_DEV uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
SP_DEV float order_key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// wave-level reductions (64 lanes)
SP_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
SP_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SP_DEV uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Inclusive prefix sum over the 64 lanes (lane l gets the sum of lanes 0..l)
// on DPP moves: shifts of 1, 2, 4, 8 inside each 16-lane row (lanes shifted
// in from outside the row read 0), then lane 15 of rows 0 and 2 added to
// rows 1 and 3, then lane 31 added to rows 2 and 3. Every lane must be active.
SP_DEV uint32_t wave_prefix_incl_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Sum and maxima over the 64 lanes with the same DPP pattern, the result
// read from lane 63 (wave-uniform). For the maxima a lane with no source lane
// keeps its own value. Every lane must be active.
SP_DEV float wave_sum_dpp(float v) {
#define SP_DPP_ADD(ctrl, rm, bc) \
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, rm, 0xf, bc))
  SP_DPP_ADD(0x111, 0xf, true);
  SP_DPP_ADD(0x112, 0xf, true);
  SP_DPP_ADD(0x114, 0xf, true);
  SP_DPP_ADD(0x118, 0xf, true);
  SP_DPP_ADD(0x142, 0xa, false);
  SP_DPP_ADD(0x143, 0xc, false);
#undef SP_DPP_ADD
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
SP_DEV float wave_max_dpp(float v) {
#define SP_DPP_MAX(ctrl, rm)                                                                     \
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), \
                                                                      __builtin_bit_cast(int, v), ctrl, rm, 0xf, false)))
  SP_DPP_MAX(0x111, 0xf);
  SP_DPP_MAX(0x112, 0xf);
  SP_DPP_MAX(0x114, 0xf);
  SP_DPP_MAX(0x118, 0xf);
  SP_DPP_MAX(0x142, 0xa);
  SP_DPP_MAX(0x143, 0xc);
#undef SP_DPP_MAX
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
SP_DEV uint32_t wave_max_u32_dpp(uint32_t v) {
#define SP_DPP_UMAX(ctrl, rm) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, ctrl, rm, 0xf, false))
  SP_DPP_UMAX(0x111, 0xf);
  SP_DPP_UMAX(0x112, 0xf);
  SP_DPP_UMAX(0x114, 0xf);
  SP_DPP_UMAX(0x118, 0xf);
  SP_DPP_UMAX(0x142, 0xa);
  SP_DPP_UMAX(0x143, 0xc);
#undef SP_DPP_UMAX
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Maximum and sum over the lanes l, l^16, l^32, l^48 (the same position in
// the four 16-lane rows) with the gfx950 lane swaps: permlane16_swap of a
// value with itself gives every lane the row-0/row-1 (row-2/row-3) pair's two
// values, permlane32_swap the two halves'. Each lane combines the same two
// operands in the same order, so all four lanes end with identical bits.
SP_DEV float rows4_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SP_DEV float rows4_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Number of active lanes below this one whose predicate is set.
SP_DEV uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

SP_DEV uint64_t ballot(bool p) { return __ballot(p); }

}  // namespace sp
