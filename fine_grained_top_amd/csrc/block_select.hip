// Block routing: pooled block keys, per-row block scores, certified top-nb.
//
//  pool:  ksum[b,hk,beta,c] = sum_{t<bs} k[b,hk,bs*beta+t,c]   (float32)
//         amax[b,hk,beta]   = max_c sum_t |k[..]|               (error-bound input)
//         ksum64, the same sums in float64 with an exactness flag per block
//  select: the eligible blocks are the complete past ones; score~(beta) =
//         (q . ksum[beta]) / bs in float32; the nb-th largest score t and a
//         rigorous bound eps give the band |score~ - t| <= 2 eps whose members
//         are rescored exactly (the float32 nearest to the exact mean of q.k
//         over the block); the best blocks by (exact key desc, block asc) are
//         kept and written in ascending block order.
#include "common.h"
#include "exact.h"
#include "internal.h"

namespace sp {

constexpr int kBsThreads = 256;

__global__ __launch_bounds__(128) void pool_kernel(BlockSelectParams p) {
  const int nbk = p.ctx / p.bs;
  const int beta = blockIdx.x % nbk;
  const int hk = (blockIdx.x / nbk) % p.Hkv;
  const int b = blockIdx.x / (nbk * p.Hkv);
  const int c = threadIdx.x;
  float s = 0.f, sa = 0.f;
  double s64 = 0.0;
  bool exact = true;
  if (c < p.d) {
    const int64_t base = b * p.k.s[0] + hk * p.k.s[1] + (int64_t)beta * p.bs * p.k.s[2] + c;
    for (int t = 0; t < p.bs; ++t) {
      const float x = p.k.dt == DT_F32 ? ((const float*)p.k.p)[base + t * p.k.s[2]]
                                        : bf16_to_f32(((const uint16_t*)p.k.p)[base + t * p.k.s[2]]);
      s += x;
      sa += fabsf(x);
      // error-free transformation (TwoSum): the float64 sum is exact while every error term is 0
      const double xs = (double)x, sn = s64 + xs;
      const double bb = sn - s64;
      const double err = (s64 - (sn - bb)) + (xs - bb);
      exact &= err == 0.0;
      s64 = sn;
    }
    const int64_t o = (((int64_t)b * p.Hkv + hk) * nbk + beta) * p.d + c;
    p.kbar[o] = s;
    p.kbar64[o] = s64;
    // s = hi + mid + r with |r| <= 2^-16 |s| (each part the nearest bf16 of what is left)
    const uint32_t hi = f32_to_bf16_rne(s);
    const uint32_t mid = f32_to_bf16_rne(s - bf16_to_f32(hi));
    const int64_t nall = (int64_t)p.B * p.Hkv * nbk * p.d;
    p.kb2[o] = (uint16_t)hi;
    p.kb2[nall + o] = (uint16_t)mid;
  }
  __shared__ float red[2];
  __shared__ int ex[2];
  float m = wave_max(c < p.d ? sa : 0.f);
  const bool allx = __all(exact);
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = m;
    ex[threadIdx.x >> 6] = allx ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t ob = ((int64_t)b * p.Hkv + hk) * nbk + beta;
    p.kabs[ob] = fmaxf(red[0], red[1]);
    p.kexact[ob] = (ex[0] && ex[1]) ? 1u : 0u;
  }
}

// exact block key computed by one wave: float64 partial sums over the lanes,
// certified, else the exact accumulator on lane 0. qrow holds the query row
// in type qdt (the caller's LDS copy, exact).
SP_DEV float wave_block_key(const BlockSelectParams& p, const void* qrow, int qdt, const void* kblock) {
  const int lane = threadIdx.x & 63;
  const int n = p.bs * p.d;
  double y = 0.0, A = 0.0;
  bool x = true;
  for (int e = lane; e < n; e += 64) {
    const int t = e / p.d, c = e % p.d;
    const double v = load_f64(qrow, qdt, c) * load_f64(kblock, p.k.dt, t * p.k.s[2] + c);   // exact
    xadd(y, x, v);
    A += fabs(v);
  }
  wave_xreduce(y, x, A);
  if (x) return key_of_exact(ldexp(y, -p.log2bs));
  const double g52 = 2.220446049250313e-16;
  const double e = 2.0 * (n + 72) * g52 * A + 1e-300;
  float key;
  const bool ok = certify(ldexp(y, -p.log2bs), ldexp(e, -p.log2bs), key);
  if (ok) return key;
  float slow = 0.f;
  if (lane == 0) slow = exact_block_key(qrow, qdt, kblock, p.k.dt, p.k.s[2], p.bs, p.log2bs, p.d);
  return __shfl(slow, 0, 64);
}

// The same key from the block's exact float64 key sums: (1/bs) * q . ksum,
// d products per candidate instead of bs * d; exact or certified, else the
// full sum. The flag and the sums (d <= 128: two per lane) load together.
SP_DEV float wave_block_key_sums(const BlockSelectParams& p, const void* qrow, int qdt, const double* ks64,
                                 const uint32_t* kx, const void* kblock) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const double k0 = ks64[lane];
  const double k1 = lane + 64 < p.d ? ks64[lane + 64] : 0.0;
  if (*kx != 0) {
    double y = 0.0, A = 0.0;
    bool x = true;
    const double q0 = load_f64(qrow, qdt, lane);
    xadd_prod(y, x, q0, k0);
    A += fabs(q0 * k0);
    if (lane + 64 < p.d) {
      const double q1 = load_f64(qrow, qdt, lane + 64);
      xadd_prod(y, x, q1, k1);
      A += fabs(q1 * k1);
    }
    wave_xreduce(y, x, A);
    if (x) return key_of_exact(ldexp(y, -p.log2bs));
    const double g52 = 2.220446049250313e-16;
    const double e = 2.0 * (2 * p.d + 72) * g52 * A + 1e-300;
    float key;
    if (certify(ldexp(y, -p.log2bs), ldexp(e, -p.log2bs), key)) return key;
  }
  return wave_block_key(p, qrow, qdt, kblock);
}

// want-th largest (want >= 1) of the keys k[j] on lanes set in vm[j]
// (slot j of lane l holds element 64 j + l; the set must have >= want
// members): radix select, 8 bits a pass, on a per-wave LDS histogram of 256
// 16-bit bins packed two to a word (128 words; counts stay below 2^16).
// Wave-uniform result.
template <int KPL>
SP_DEV uint32_t wave_kth_largest(const uint32_t (&k)[KPL], const uint64_t (&vm)[KPL], int n, uint32_t want,
                                 uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0;
#pragma unroll
  for (int shift = 24; shift >= 0; shift -= 8) {
    *(u32x2*)(hist + 2 * lane) = u32x2{0u, 0u};
    __builtin_amdgcn_wave_barrier();
    const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (j * 64 >= n) break;
      if (((vm[j] >> lane) & 1) && (k[j] & hmask) == prefix) {
        const uint32_t dgt = (k[j] >> shift) & 255u;
        atomicAdd(&hist[dgt >> 1], 1u << ((dgt & 1u) << 4));
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lane l owns bins 4l .. 4l+3
    const u32x2 hw = *(const u32x2*)(hist + 2 * lane);
    const uint32_t h0 = hw[0] & 0xFFFFu, h1 = hw[0] >> 16, h2 = hw[1] & 0xFFFFu, h3 = hw[1] >> 16;
    const uint32_t c = h0 + h1 + h2 + h3;
    // members with a digit in a higher lane's bins
    const uint32_t pin = wave_prefix_incl_u32(c);
    const uint32_t above0 = (uint32_t)__builtin_amdgcn_readlane((int)pin, 63) - pin;
    // the bin where the count from the top reaches want
    uint32_t dg = 0, above = 0;
    if (above0 + h3 >= want) { dg = 3; above = above0; }
    else if (above0 + h3 + h2 >= want) { dg = 2; above = above0 + h3; }
    else if (above0 + h3 + h2 + h1 >= want) { dg = 1; above = above0 + h3 + h2; }
    else { dg = 0; above = above0 + h3 + h2 + h1; }
    const uint64_t hit = ballot(above0 < want && want <= above0 + c);
    const int src = (int)__builtin_ctzll(hit);
    const uint32_t digit = 4u * (uint32_t)src + (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
    want -= (uint32_t)__builtin_amdgcn_readlane((int)above, src);
    prefix |= digit << shift;
    __builtin_amdgcn_wave_barrier();
  }
  return prefix;
}

// Select, one workgroup per tile of RB consecutive query rows of one (b, h):
//  phase 1: score~[rr][beta] = (q_rr . ksum[beta]) / bs for every block any row
//           of the tile may see, into LDS as order keys. bf16 q: MFMA tiles of
//           16 rows x 16 blocks, the key sums as two bf16 parts, the q tile in
//           registers (and copied to LDS for phase 2); float32 q: one thread
//           per block reusing its key sum across the RB rows;
//  phase 2: one wave per row: the nb-th largest score (radix select), the
//           band, exact keys of the band, the R best of the band, ordered output.
template <int KPL, bool MFMA>
__global__ __launch_bounds__(kBsThreads) __attribute__((amdgpu_waves_per_eu(4))) void block_select_kernel(BlockSelectParams p, int ntile) {
  constexpr int RB = 128 / KPL;   // rows per tile: 16, 8, 4 for up to 512, 1024, 2048 blocks
  extern __shared__ __align__(16) unsigned char smem[];
  const int nbk = p.ctx / p.bs;
  // q rows of the tile: [RB][d] bf16 (MFMA) or float32
  f32x4* qs = (f32x4*)smem;
  uint16_t* qb = (uint16_t*)smem;
  uint32_t* sk = (uint32_t*)(smem + RB * p.d * (MFMA ? 2 : 4));   // [RB][nbk]
  __shared__ float qn[RB];
  __shared__ float fred[4];
  // per wave: the radix histogram, which the band lists (64 indices, 64 keys) reuse
  __shared__ __align__(16) uint32_t whist[4][128];

  // blockIdx -> tile: a contiguous range of tiles per XCD (dispatch round-robins
  // workgroups over the 8 XCDs), so one XCD's L2 holds few heads' key sums
  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
  const int tile = wg % ntile;
  const int h = (wg / ntile) % p.Hq;
  const int b = wg / (ntile * p.Hq);
  const int r0 = tile * RB;
  const int nrows = min(RB, p.Nq - r0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hk = h / (p.Hq / p.Hkv);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  auto ne_of = [&](int rr) {
    const int pos = L - p.Nq + r0 + rr;
    return pos >= 0 ? min((pos + 1) / p.bs, nbk) : 0;
  };
  const int neMax = ne_of(nrows - 1);
  const int nb = p.nb;
  const int esz = p.q.dt == DT_F32 ? 4 : 2;
  const int d4 = p.d >> 2;

  if (neMax > nb) {
    const float* ka = p.kabs + ((int64_t)b * p.Hkv + hk) * nbk;
    const float inv = ldexpf(1.0f, -p.log2bs);
    float amax = 0.f;
    if (MFMA) {
      // S[16 rows][16 blocks] = Q K^T on v_mfma_f32_16x16x32_bf16 over the two
      // bf16 parts of the block sums: A = q rows (lane: row l%16, dims
      // 32 st + 8(l/16) ..+7), B = parts (lane: block l%16, same dims),
      // D: lane block l%16, rows 4(l/16)+v
      const int64_t nall = (int64_t)p.B * p.Hkv * nbk * p.d;
      const uint16_t* kp = p.kb2 + ((int64_t)b * p.Hkv + hk) * nbk * p.d;
      const int m16 = lane & 15, kg = lane >> 4;
      const int nst = p.d >> 5;
      // block 1-norm bounds: issued first, consumed after the tiles (nbk <= 512)
      const float ka0 = tid < neMax ? ka[tid] : 0.f;
      const float ka1 = tid + kBsThreads < neMax ? ka[tid + kBsThreads] : 0.f;
      u32x4 qa[4];
      {
        const uint16_t* qr = (const uint16_t*)p.q.p + b * p.q.s[0] + h * p.q.s[1] +
                             (int64_t)(r0 + min(m16, nrows - 1)) * p.q.s[2] + 8 * kg;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (st < nst) v = *(const u32x4*)(qr + 32 * st);   // rows are 16-byte aligned (checked at the boundary)
          if (m16 >= nrows) v = u32x4{0u, 0u, 0u, 0u};
          qa[st] = v;
        }
      }
      u32x4 Bc[2][4], Bn[2][4];
      auto loadB = [&](u32x4 (&Bt)[2][4], int bt) {
        const int blk = 16 * bt + m16;
        const uint16_t* src = kp + (int64_t)(blk < neMax ? blk : neMax - 1) * p.d + 8 * kg;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (st < nst) {
            Bt[0][st] = *(const u32x4*)(src + 32 * st);
            Bt[1][st] = *(const u32x4*)(src + nall + 32 * st);
          }
        }
      };
      if (16 * wid < neMax) loadB(Bc, wid);
      // the q tile to LDS for phase 2 (wave 0) and the row 1-norms
      float a1 = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st < nst) {
          if (wid == 0) *(u32x4*)(qb + m16 * p.d + 32 * st + 8 * kg) = qa[st];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a1 += fabsf(bf16_to_f32(qa[st][e] & 0xFFFFu)) + fabsf(bf16_to_f32(qa[st][e] >> 16));
        }
      }
      a1 += __shfl_xor(a1, 16, 64);
      a1 += __shfl_xor(a1, 32, 64);
      if (wid == 0 && lane < RB) qn[lane] = a1;
      for (int bt = wid; 16 * bt < neMax; bt += 4) {
        const bool more = 16 * (bt + 4) < neMax;
        if (more) loadB(Bn, bt + 4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (st < nst) {
            const bf16x8 A = __builtin_bit_cast(bf16x8, qa[st]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, Bc[0][st]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, Bc[1][st]), acc, 0, 0, 0);
          }
        }
        const int blk = 16 * bt + m16;
        if (blk < neMax) {
#pragma unroll
          for (int v = 0; v < 4; ++v) sk[(4 * kg + v) * nbk + blk] = f32_order_key(acc[v] * inv);
        }
        if (more) {
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            Bc[0][st] = Bn[0][st];
            Bc[1][st] = Bn[1][st];
          }
        }
      }
      amax = fmaxf(ka0, ka1);
    } else {
      // q rows of the tile -> LDS, with their 1-norms
      for (int rr = wid; rr < RB; rr += 4) {
        const char* qrow = (const char*)p.q.p + (b * p.q.s[0] + h * p.q.s[1] + (int64_t)(r0 + rr) * p.q.s[2]) * esz;
        float a = 0.f;
        for (int c = lane; c < p.d; c += 64) {
          float x = 0.f;
          if (rr < nrows)
            x = p.q.dt == DT_F32 ? ((const float*)qrow)[c] : bf16_to_f32(((const uint16_t*)qrow)[c]);
          ((float*)qs)[rr * p.d + c] = x;
          a += fabsf(x);
        }
        a = wave_sum(a);
        if (lane == 0) qn[rr] = a;
      }
      __syncthreads();
      const float* kb = p.kbar + ((int64_t)b * p.Hkv + hk) * nbk * p.d;
      for (int beta = tid; beta < neMax; beta += kBsThreads) {
        const f32x4* kr = (const f32x4*)(kb + (int64_t)beta * p.d);
        float acc[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) acc[rr] = 0.f;
        for (int c4 = 0; c4 < d4; c4 += 4) {
          f32x4 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = kr[c4 + u];
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f32x4 qv = qs[rr * d4 + c4 + u];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[rr] = fmaf(qv[e], v[u][e], acc[rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) sk[rr * nbk + beta] = f32_order_key(acc[rr] * inv);
        amax = fmaxf(amax, ka[beta]);
      }
    }
    amax = wave_max(amax);
    if (lane == 0) fred[wid] = amax;
  } else if (lane == 0) {
    fred[wid] = 0.f;
  }
  __syncthreads();
  const float amax = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
  // rigorous bound on |score~ - key| per unit of |q|_1 (amax covers every block of the tile)
  const double uu = 1.0 / 8388608.0;
  auto gam = [&](double n) { return n * uu / (1.0 - n * uu); };
  // float32 sums (bs terms), then either FMA chains of d products, or MFMA
  // accumulation of the 2 d exact products with the bf16 parts hi + mid of
  // each sum (|hi| + |mid| <= (1 + 2^-6) |sum|, the remainder below 2^-16 |sum|)
  const double gb = 1.0 + gam(p.bs + 2);
  const double C = MFMA ? 1.25 * (gam(p.bs + 2) + gb / 65536.0 + gam(2 * p.d + 2) * (1.0 + 1.0 / 64.0) * gb + uu)
                        : 1.25 * (gam(p.bs + 2) + gam(p.d + 2) * gb + uu);
  const int ksz = p.k.dt == DT_F32 ? 4 : 2;

  uint32_t* hist = whist[wid];
  uint32_t* bl_i = hist;        // band lists: used only while no radix select runs
  uint32_t* bl_k = hist + 64;
  for (int rr = wid; rr < nrows; rr += 4) {
    const int r = r0 + rr;
    const int ne = __builtin_amdgcn_readfirstlane(ne_of(rr));
    int32_t* out = p.out + b * p.os[0] + h * p.os[1] + (int64_t)r * p.os[2];
    const int64_t crow = ((int64_t)b * p.Hq + h) * p.Nq + r;
    if (ne <= nb) {
      for (int i = lane; i < nb; i += 64) out[i] = i < ne ? i : -1;
      if (p.count && lane == 0) p.count[crow] = ne;
      continue;
    }
    uint32_t* wrow = sk + rr * nbk;
    uint32_t kr[KPL];
    uint64_t vm[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int i = j * 64 + lane;
      kr[j] = i < ne ? wrow[i] : 0u;
      vm[j] = ballot(i < ne);
    }
    const uint32_t t = wave_kth_largest<KPL>(kr, vm, ne, (uint32_t)nb, hist);
    const float eps = (float)(C * (double)qn[rr] * (double)amax * ldexp(1.0, -p.log2bs) * (1 + 1e-6) + 1e-30);
    const float tf = order_key_f32(t);
    const float E = 2.0f * eps * 1.0001f + 1e-30f;
    const uint32_t klo = f32_order_key(nextafterf(tf - E, -INFINITY));
    const uint32_t khi = f32_order_key(nextafterf(tf + E, INFINITY));
    uint64_t bm[KPL];
    int n_in = 0, nbd = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      bm[j] = vm[j] & ballot(kr[j] >= klo && kr[j] <= khi);
      n_in += __popcll(vm[j] & ballot(kr[j] > khi));
      nbd += __popcll(bm[j]);
    }
    // exact keys of the band (ascending block order), written over the scores
    // in LDS by every lane; the first 64 also into the wave's band list
    const void* qrow = MFMA ? (const void*)(qb + rr * p.d) : (const void*)((const float*)qs + rr * p.d);
    const int qdt = MFMA ? DT_BF16 : DT_F32;
    int e = 0;
    for (int j = 0; j * 64 < ne; ++j) {
      const int i = j * 64 + lane;
      const uint32_t kk = i < ne ? wrow[i] : 0u;
      uint64_t m = ballot(i < ne && kk >= klo && kk <= khi);
      while (m) {
        const int beta = j * 64 + __builtin_ctzll(m);
        m &= m - 1;
        const char* kblk = (const char*)p.k.p + (b * p.k.s[0] + hk * p.k.s[1] + (int64_t)beta * p.bs * p.k.s[2]) * ksz;
        const int64_t ob = ((int64_t)b * p.Hkv + hk) * nbk + beta;
        const float key = wave_block_key_sums(p, qrow, qdt, p.kbar64 + ob * p.d, p.kexact + ob, kblk);
        const uint32_t ok = f32_order_key(__builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, key))));
        wrow[beta] = ok;
        if (e < 64 && lane == 0) {
          bl_i[e] = beta;
          bl_k[e] = ok;
        }
        ++e;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // the R best of the band by (exact key desc, block asc) get the mark ~0,
    // the others 0: afterwards "selected" is "mark or score above the band"
    const int R = nb - n_in;
    if (nbd <= 64) {
      const uint32_t ke = lane < nbd ? bl_k[lane] : 0u;
      int rank = 0;
      for (int f = 0; f < nbd; ++f) {
        const uint32_t kf = (uint32_t)__builtin_amdgcn_readlane((int)ke, f);
        rank += (kf > ke || (kf == ke && f < lane)) ? 1 : 0;
      }
      if (lane < nbd) wrow[bl_i[lane]] = rank < R ? ~0u : 0u;
    } else {
      uint32_t ex[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) ex[j] = ((bm[j] >> lane) & 1) ? wrow[j * 64 + lane] : 0u;
      const uint32_t tb = wave_kth_largest<KPL>(ex, bm, ne, (uint32_t)R, hist);
      int gt = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) gt += __popcll(bm[j] & ballot(ex[j] > tb));
      const int need = R - gt;
      int ties = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        if (j * 64 >= ne) break;
        const bool band = (bm[j] >> lane) & 1;
        const uint64_t tm = bm[j] & ballot(ex[j] == tb);
        const int trank = ties + (int)lanes_below(tm);
        if (band) wrow[j * 64 + lane] = (ex[j] > tb || (ex[j] == tb && trank < need)) ? ~0u : 0u;
        ties += __popcll(tm);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ordered output
    int opos = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (j * 64 >= ne) break;
      const int i = j * 64 + lane;
      const uint32_t kk = ((bm[j] >> lane) & 1) ? wrow[i] : kr[j];
      const bool sel = i < ne && kk > khi;
      const uint64_t smk = ballot(sel);
      const int o = opos + (int)lanes_below(smk);
      if (sel && o < nb) out[o] = i;
      opos += __popcll(smk);
    }
    if (p.count && lane == 0) p.count[crow] = nb;
  }
}

size_t block_select_ws_bytes(int B, int Hkv, int ctx, int d, int bs) {
  const size_t nbk = ctx / bs;
  // kbar64 (2 floats each), kbar, kabs, kexact, then the two bf16 parts (256-byte aligned)
  return (size_t)B * Hkv * nbk * (3 * d + 2) * sizeof(float) + 256 + (size_t)B * Hkv * nbk * d * 2 * 2;
}

hipError_t launch_block_select(const BlockSelectParams& p, hipStream_t st) {
  const int nbk = p.ctx / p.bs;
  hipLaunchKernelGGL(pool_kernel, dim3(p.B * p.Hkv * nbk), dim3(128), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int kpl = nbk <= 512 ? 8 : nbk <= 1024 ? 16 : 32;
  const int rb = 128 / kpl;
  const int ntile = (p.Nq + rb - 1) / rb;
  const bool mfma = kpl == 8 && p.q.dt == DT_BF16;
  const size_t lds = (size_t)rb * p.d * (mfma ? 2 : 4) + (size_t)rb * nbk * 4;
  const dim3 grid(p.B * p.Hq * ntile);
  if (mfma)
    hipLaunchKernelGGL((block_select_kernel<8, true>), grid, dim3(kBsThreads), lds, st, p, ntile);
  else if (kpl == 8)
    hipLaunchKernelGGL((block_select_kernel<8, false>), grid, dim3(kBsThreads), lds, st, p, ntile);
  else if (kpl == 16)
    hipLaunchKernelGGL((block_select_kernel<16, false>), grid, dim3(kBsThreads), lds, st, p, ntile);
  else
    hipLaunchKernelGGL((block_select_kernel<32, false>), grid, dim3(kBsThreads), lds, st, p, ntile);
  return hipGetLastError();
}

}  // namespace sp
