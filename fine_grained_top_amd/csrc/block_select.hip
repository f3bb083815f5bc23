// Block routing: pooled block keys, per-row block scores, certified top-nb.
//
//  pool:  ksum[b,hk,beta,c] = sum_{t<bs} k[b,hk,bs*beta+t,c]   (float32)
//         amax[b,hk,beta]   = max_c sum_t |k[..]|               (error-bound input)
//  select (one workgroup per (b, h, r)): the eligible blocks are the complete
//         past ones; score~(beta) = (q . ksum[beta]) / bs in float32; the
//         nb-th largest score t and a rigorous bound eps give the band
//         |score~ - t| <= 2 eps whose members are rescored exactly (the
//         float32 nearest to the exact mean of q.k over the block) by one
//         wave each; the best blocks by (exact key desc, block asc) are kept
//         and written in ascending block order.
#include "common.h"
#include "exact.h"
#include "internal.h"
#include "rowselect.h"

namespace sp {

constexpr int kBsThreads = 256;
constexpr int kMaxBlocks = 2048;

__global__ __launch_bounds__(128) void pool_kernel(BlockSelectParams p) {
  const int nbk = p.ctx / p.bs;
  const int beta = blockIdx.x % nbk;
  const int hk = (blockIdx.x / nbk) % p.Hkv;
  const int b = blockIdx.x / (nbk * p.Hkv);
  const int c = threadIdx.x;
  float s = 0.f, sa = 0.f;
  if (c < p.d) {
    const int64_t base = b * p.k.s[0] + hk * p.k.s[1] + (int64_t)beta * p.bs * p.k.s[2] + c;
    for (int t = 0; t < p.bs; ++t) {
      const float x = p.k.dt == DT_F32 ? ((const float*)p.k.p)[base + t * p.k.s[2]]
                                        : bf16_to_f32(((const uint16_t*)p.k.p)[base + t * p.k.s[2]]);
      s += x;
      sa += fabsf(x);
    }
    p.kbar[(((int64_t)b * p.Hkv + hk) * nbk + beta) * p.d + c] = s;
  }
  __shared__ float red[2];
  float m = wave_max(c < p.d ? sa : 0.f);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) p.kabs[((int64_t)b * p.Hkv + hk) * nbk + beta] = fmaxf(red[0], red[1]);
}

// exact block key computed by one wave: float64 partial sums over the lanes,
// certified, else the exact accumulator on lane 0.
SP_DEV float wave_block_key(const BlockSelectParams& p, const void* qrow, const void* kblock) {
  const int lane = threadIdx.x & 63;
  const int n = p.bs * p.d;
  double y = 0.0, A = 0.0;
  for (int e = lane; e < n; e += 64) {
    const int t = e / p.d, c = e % p.d;
    const double v = load_f64(qrow, p.q.dt, c) * load_f64(kblock, p.k.dt, t * p.k.s[2] + c);
    y += v;
    A += fabs(v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    y += __shfl_xor(y, o, 64);
    A += __shfl_xor(A, o, 64);
  }
  const double g52 = 2.220446049250313e-16;
  const double e = 2.0 * (n + 72) * g52 * A + 1e-300;
  float key;
  const bool ok = certify(ldexp(y, -p.log2bs), ldexp(e, -p.log2bs), key);
  if (ok) return key;
  float slow = 0.f;
  if (lane == 0) slow = exact_block_key(qrow, p.q.dt, kblock, p.k.dt, p.k.s[2], p.bs, p.log2bs, p.d);
  return __shfl(slow, 0, 64);
}

__global__ __launch_bounds__(kBsThreads) void block_select_kernel(BlockSelectParams p) {
  constexpr int T = kBsThreads;
  __shared__ uint32_t keys[kMaxBlocks];
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t band_b[kMaxBlocks];
  __shared__ uint32_t band_k[kMaxBlocks];
  __shared__ float qs[128];
  __shared__ uint32_t sc[16];
  __shared__ uint32_t run[4];
  __shared__ float fred[8];

  const int row = blockIdx.x;
  const int r = row % p.Nq;
  const int h = (row / p.Nq) % p.Hq;
  const int b = row / (p.Nq * p.Hq);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int hk = h / (p.Hq / p.Hkv);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  const int nbk = p.ctx / p.bs;
  const int ne = pos >= 0 ? min((pos + 1) / p.bs, nbk) : 0;
  const int nb = p.nb;
  int32_t* out = p.out + b * p.os[0] + h * p.os[1] + r * p.os[2];

  if (ne <= nb) {
    for (int i = tid; i < nb; i += T) out[i] = i < ne ? i : -1;
    if (p.count && tid == 0) p.count[((int64_t)b * p.Hq + h) * p.Nq + r] = ne;
    return;
  }
  const int esz = p.q.dt == DT_F32 ? 4 : 2;
  const char* qrow = (const char*)p.q.p + (b * p.q.s[0] + h * p.q.s[1] + r * p.q.s[2]) * esz;
  float qa = 0.f;
  for (int c = tid; c < p.d; c += T) {
    const float x = p.q.dt == DT_F32 ? ((const float*)qrow)[c] : bf16_to_f32(((const uint16_t*)qrow)[c]);
    qs[c] = x;
    qa += fabsf(x);
  }
  qa = wave_sum(qa);
  if (lane == 0) fred[wid] = qa;
  __syncthreads();
  const float qnorm1 = fred[0] + fred[1] + fred[2] + fred[3];
  __syncthreads();

  const float* kb = p.kbar + ((int64_t)b * p.Hkv + hk) * nbk * p.d;
  const float* ka = p.kabs + ((int64_t)b * p.Hkv + hk) * nbk;
  const float inv = ldexpf(1.0f, -p.log2bs);
  float amax = 0.f;
  for (int beta = tid; beta < ne; beta += T) {
    const f32x4* kr = (const f32x4*)(kb + (int64_t)beta * p.d);   // rows of d floats, 16-byte aligned
    float s = 0.f;
    for (int c4 = 0; c4 < p.d / 4; c4 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = kr[c4 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(qs[4 * (c4 + u) + e], v[u][e], s);
    }
    keys[beta] = f32_order_key(s * inv);
    amax = fmaxf(amax, ka[beta]);
  }
  amax = wave_max(amax);
  if (lane == 0) fred[wid] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));

  uint32_t t, above;
  radix_select<T>(ne, (uint32_t)nb, [&](int i, uint32_t& k) { k = keys[i]; return true; }, hist, sc, t,
                  above);
  // rigorous bound on |score~ - key|
  const double u = 1.0 / 8388608.0;
  auto gam = [&](double n) { return n * u / (1.0 - n * u); };
  const double C = 1.25 * (gam(p.bs + 2) + gam(p.d + 2) * (1.0 + gam(p.bs + 2)) + u);
  const float eps = (float)(C * (double)qnorm1 * (double)amax * (double)inv * (1 + 1e-6) + 1e-30);
  const float tf = order_key_f32(t);
  const float E = 2.0f * eps * 1.0001f + 1e-30f;
  const uint32_t klo = f32_order_key(nextafterf(tf - E, -INFINITY));
  const uint32_t khi = f32_order_key(nextafterf(tf + E, INFINITY));

  // ordered pass: count blocks above the band, list the band (ascending)
  if (tid == 0) { run[0] = 0; run[1] = 0; }
  __syncthreads();
  for (int base = 0; base < ne; base += T) {
    const int i = base + tid;
    bool in = false, bd = false;
    if (i < ne) {
      in = keys[i] > khi;
      bd = keys[i] >= klo && keys[i] <= khi;
    }
    uint32_t nin, nbd;
    const uint32_t bpos = block_prefix<T>(bd, sc, nbd);
    block_prefix<T>(in, sc, nin);
    if (bd) band_b[run[1] + bpos] = i;
    __syncthreads();
    if (tid == 0) { run[0] += nin; run[1] += nbd; }
    __syncthreads();
  }
  const uint32_t n_in = run[0], n_band = run[1];
  // exact keys of the band, one wave per block
  const int ksz = p.k.dt == DT_F32 ? 4 : 2;
  for (uint32_t e = wid; e < n_band; e += T / 64) {
    const int beta = band_b[e];
    const char* kblk = (const char*)p.k.p +
                       (b * p.k.s[0] + hk * p.k.s[1] + (int64_t)beta * p.bs * p.k.s[2]) * ksz;
    const float key = wave_block_key(p, qrow, kblk);
    if (lane == 0) band_k[e] = f32_order_key(key);
  }
  __syncthreads();
  // keep the R best of the band by (exact key desc, block asc): rank by counting
  const uint32_t R = (uint32_t)nb - n_in;
  for (uint32_t e = tid; e < n_band; e += T) {
    const uint32_t ke = band_k[e];
    uint32_t rank = 0;
    for (uint32_t f = 0; f < n_band; ++f) {
      const uint32_t kf = band_k[f];
      rank += (kf > ke || (kf == ke && f < e)) ? 1u : 0u;
    }
    if (rank < R) band_b[e] |= 0x80000000u;
  }
  __syncthreads();
  // ordered output
  if (tid == 0) { run[0] = 0; run[1] = 0; }
  __syncthreads();
  for (int base = 0; base < ne; base += T) {
    const int i = base + tid;
    bool sel = false, bd = false;
    if (i < ne) {
      sel = keys[i] > khi;
      bd = keys[i] >= klo && keys[i] <= khi;
    }
    uint32_t nbd, nsel;
    const uint32_t brank = run[1] + block_prefix<T>(bd, sc, nbd);
    if (bd) sel = (band_b[brank] & 0x80000000u) != 0;
    const uint32_t opos = run[0] + block_prefix<T>(sel, sc, nsel);
    if (sel && opos < (uint32_t)nb) out[opos] = i;
    __syncthreads();
    if (tid == 0) { run[0] += nsel; run[1] += nbd; }
    __syncthreads();
  }
  if (p.count && tid == 0) p.count[((int64_t)b * p.Hq + h) * p.Nq + r] = nb;
}

size_t block_select_ws_bytes(int B, int Hkv, int ctx, int d, int bs) {
  const size_t nbk = ctx / bs;
  return (size_t)B * Hkv * nbk * (d + 1) * sizeof(float);
}

hipError_t launch_block_select(const BlockSelectParams& p, hipStream_t st) {
  const int nbk = p.ctx / p.bs;
  hipLaunchKernelGGL(pool_kernel, dim3(p.B * p.Hkv * nbk), dim3(128), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_select_kernel, dim3(p.B * p.Hq * p.Nq), dim3(kBsThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sp
