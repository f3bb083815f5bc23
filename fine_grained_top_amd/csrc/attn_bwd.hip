// Tiled backward of the contiguous fixed patterns (dense causal, sliding
// window + global tokens), bf16, d = 128.
//
// One workgroup = 64 query rows of one (request, head), the key tiles of 64
// keys visited as by the forward tile kernel (global tiles and the window's
// band, or every past tile). Per key tile, with Q, dO, K, V tiles in LDS and
// each thread holding a 4 x 4 block of (row, key) pairs in registers:
//   S = Q K^T, dP = dO V^T (128-term dot products),
//   P = exp(S * scale - lse) on visible pairs, dS = P (dP - D) * scale,
// then with 4 x 8 blocks of outputs per thread:
//   dQ += dS K     (kept in registers over the key tiles),
//   dK  = dS^T Q,  dV = P^T dO  (this query tile's share, added to the
//   key tile's rows with one float atomic per element).
// D = rowsum(dO * O) per row. Float32 throughout; bf16 inputs are exact.
#include "common.h"
#include "internal.h"

namespace sp {

constexpr int kBT = 64;         // rows per query tile, keys per key tile
constexpr int kBD = 128;        // head dim
constexpr int kBQs = kBD + 2;   // bf16 row stride of the Q/K/V tiles: 65 words, so rows fall in distinct banks
constexpr int kBPs = kBT + 1;   // float row stride of the P and dS tiles

struct BwdSmem {
  uint16_t q[kBT * kBQs];
  uint16_t k[kBT * kBQs];
  uint16_t v[kBT * kBQs];
  float dO[kBT * (kBD + 1)];
  float P[kBT * kBPs];
  float dS[kBT * kBPs];
  float D[kBT], lse[kBT];
  uint32_t tiles[64];
};

SP_DEV float bfl(const uint16_t* t, int i) { return bf16_to_f32(t[i]); }

__global__ __launch_bounds__(256) void attn_bwd_tile_kernel(AttnParams a, AttnBwd g) {
  __shared__ BwdSmem sm;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int kvh = h / (a.Hq / a.Hkv);
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int q0 = qt * kBT;
  const int pbase = L - a.Nq;
  const int nrows = min(kBT, a.Nq - q0);
  const int prow_first = pbase + q0, prow_last = pbase + q0 + nrows - 1;
  const int ntiles_all = (L + kBT - 1) / kBT;

  // ---- the query tile: Q (bf16), dO, D = rowsum(dO * O), lse
  for (int e = tid; e < kBT * kBD; e += 256) {
    const int r = e >> 7, c = e & 127;
    uint16_t qv = 0;
    float dov = 0.f;
    if (r < nrows) {
      qv = ((const uint16_t*)a.q.p)[b * a.q.s[0] + h * a.q.s[1] + (int64_t)(q0 + r) * a.q.s[2] + c];
      dov = g.dO[b * g.dos[0] + h * g.dos[1] + (int64_t)(q0 + r) * g.dos[2] + c];
    }
    sm.q[r * kBQs + c] = qv;
    sm.dO[r * (kBD + 1) + c] = dov;
  }
  if (tid < 64) sm.tiles[tid] = 0;
  __syncthreads();
  {
    // D: four threads per row, 32 dims each
    const int r = tid >> 2, part = tid & 3;
    float s = 0.f;
    if (r < nrows) {
      const float* orow = g.o + b * g.os[0] + h * g.os[1] + (int64_t)(q0 + r) * g.os[2];
      for (int c = 32 * part; c < 32 * part + 32; ++c) s = fmaf(sm.dO[r * (kBD + 1) + c], orow[c], s);
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) {
      sm.D[r] = s;
      sm.lse[r] = r < nrows ? g.lse[((int64_t)b * a.Hq + h) * a.Nq + q0 + r] : -INFINITY;
    }
  }
  // ---- key tiles any row of the tile can see
  const int last_tile = min(ntiles_all - 1, prow_last / kBT);
  if (a.mode == 0) {
    for (int t = tid; t <= last_tile; t += 256) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
  } else {
    const int gt = (min(a.n_global, L) + kBT - 1) / kBT;
    const int wt = max(0, prow_first - a.window + 1) / kBT;
    for (int t = tid; t <= last_tile; t += 256)
      if (t < gt || t >= wt) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
  }
  __syncthreads();

  // thread blocks: pairs rows 4*(tid/16) + i, keys tid%16 + 16*j (keys 16 apart
  // fall in distinct LDS banks); outputs rows/keys 4*(tid/16) + i, dims
  // 8*(tid%16) + e
  const int pr = 4 * (tid >> 4), pk = tid & 15;
  const int orow = 4 * (tid >> 4), odim = 8 * (tid & 15);
  float dq[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) dq[i][e] = 0.f;
  const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.s[0] + kvh * a.k.s[1];
  const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.s[0] + kvh * a.v.s[1];
  float* dkb = g.dk + b * g.dks[0] + kvh * g.dks[1];
  float* dvb = g.dv + b * g.dvs[0] + kvh * g.dvs[1];

  for (int w = 0; w <= (last_tile >> 5) && last_tile >= 0; ++w) {
    uint32_t bits = sm.tiles[w];
    while (bits) {
      const int t = 32 * w + __builtin_ctz(bits);
      bits &= bits - 1;
      const int j0 = t * kBT;
      // stage K and V tiles (keys past L read as row L-1, masked below)
      for (int e = tid; e < kBT * kBD / 8; e += 256) {
        const int kr = e >> 4, c8 = (e & 15) * 8;
        const int j = min(j0 + kr, L - 1);
        const u32x4 kv = *(const u32x4*)(kbase + (int64_t)j * a.k.s[2] + c8);
        const u32x4 vv = *(const u32x4*)(vbase + (int64_t)j * a.v.s[2] + c8);
        uint32_t* kd = (uint32_t*)&sm.k[kr * kBQs + c8];
        uint32_t* vd = (uint32_t*)&sm.v[kr * kBQs + c8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kd[u] = kv[u];
          vd[u] = vv[u];
        }
      }
      __syncthreads();
      // S and dP for the thread's 4 x 4 block
      float s[4][4], dp[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s[i][jj] = dp[i][jj] = 0.f;
      for (int c = 0; c < kBD; c += 2) {
        float qa[4][2], oa[4][2], ka[4][2], va[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t qw = *(const uint32_t*)&sm.q[(pr + i) * kBQs + c];
          qa[i][0] = bf16_to_f32(qw & 0xFFFFu);
          qa[i][1] = bf16_to_f32(qw >> 16);
          oa[i][0] = sm.dO[(pr + i) * (kBD + 1) + c];
          oa[i][1] = sm.dO[(pr + i) * (kBD + 1) + c + 1];
          const uint32_t kw = *(const uint32_t*)&sm.k[(pk + 16 * i) * kBQs + c];
          const uint32_t vw = *(const uint32_t*)&sm.v[(pk + 16 * i) * kBQs + c];
          ka[i][0] = bf16_to_f32(kw & 0xFFFFu);
          ka[i][1] = bf16_to_f32(kw >> 16);
          va[i][0] = bf16_to_f32(vw & 0xFFFFu);
          va[i][1] = bf16_to_f32(vw >> 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            s[i][jj] = fmaf(qa[i][0], ka[jj][0], s[i][jj]);
            s[i][jj] = fmaf(qa[i][1], ka[jj][1], s[i][jj]);
            dp[i][jj] = fmaf(oa[i][0], va[jj][0], dp[i][jj]);
            dp[i][jj] = fmaf(oa[i][1], va[jj][1], dp[i][jj]);
          }
      }
      // P and dS on visible pairs
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = pr + i;
        const int prow = pbase + q0 + r;
        const float lr = sm.lse[r], Dr = sm.D[r];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = j0 + pk + 16 * jj;
          bool vis = r < nrows && j <= prow && lr > -INFINITY;
          if (vis && a.mode == 2) vis = j >= prow - a.window + 1 || j < a.n_global;
          const float p = vis ? expf(s[i][jj] * a.scale - lr) : 0.f;
          sm.P[r * kBPs + pk + 16 * jj] = p;
          sm.dS[r * kBPs + pk + 16 * jj] = p * (dp[i][jj] - Dr) * a.scale;
        }
      }
      __syncthreads();
      // dQ += dS K (rows orow.., dims odim..)
      for (int jj = 0; jj < kBT; ++jj) {
        float kv[8];
        const uint32_t* kw = (const uint32_t*)&sm.k[jj * kBQs + odim];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kv[2 * u] = bf16_to_f32(kw[u] & 0xFFFFu);
          kv[2 * u + 1] = bf16_to_f32(kw[u] >> 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = sm.dS[(orow + i) * kBPs + jj];
#pragma unroll
          for (int e = 0; e < 8; ++e) dq[i][e] = fmaf(d, kv[e], dq[i][e]);
        }
      }
      // dK = dS^T Q and dV = P^T dO for keys orow.., dims odim..
      float dk[4][8], dv[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) dk[i][e] = dv[i][e] = 0.f;
      for (int r = 0; r < nrows; ++r) {
        float qv[8], ov[8];
        const uint32_t* qw = (const uint32_t*)&sm.q[r * kBQs + odim];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          qv[2 * u] = bf16_to_f32(qw[u] & 0xFFFFu);
          qv[2 * u + 1] = bf16_to_f32(qw[u] >> 16);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = sm.dO[r * (kBD + 1) + odim + e];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = sm.dS[r * kBPs + orow + i], p = sm.P[r * kBPs + orow + i];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            dk[i][e] = fmaf(d, qv[e], dk[i][e]);
            dv[i][e] = fmaf(p, ov[e], dv[i][e]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + orow + i;
        if (j >= L) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (dk[i][e] != 0.f) atomicAdd(&dkb[(int64_t)j * g.dks[2] + odim + e], dk[i][e]);
          if (dv[i][e] != 0.f) atomicAdd(&dvb[(int64_t)j * g.dvs[2] + odim + e], dv[i][e]);
        }
      }
      __syncthreads();
    }
  }
  // ---- dQ
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (orow + i >= nrows) continue;
    float* dqr = g.dq + b * g.dqs[0] + h * g.dqs[1] + (int64_t)(q0 + orow + i) * g.dqs[2] + odim;
#pragma unroll
    for (int e = 0; e < 8; ++e) dqr[e] = dq[i][e];
  }
}

bool attn_bwd_tile_ok(const AttnParams& a) {
  return a.q.dt == DT_BF16 && a.d == kBD && !a.ptab && (a.mode == 0 || (a.mode == 2 && a.stride == 0)) &&
         (a.ctx + kBT - 1) / kBT <= 2048;
}

hipError_t launch_attn_bwd_tile(const AttnParams& a, const AttnBwd& g, hipStream_t st) {
  dim3 grid((a.Nq + kBT - 1) / kBT, a.Hq, a.B);
  hipLaunchKernelGGL(attn_bwd_tile_kernel, grid, dim3(256), 0, st, a, g);
  return hipGetLastError();
}

}  // namespace sp
