// Tiled backward of the contiguous fixed patterns (dense causal, sliding
// window + global tokens), bf16, d = 128.
//
// One workgroup = 64 query rows of one (request, head), the key tiles of 64
// keys visited as by the forward tile kernel (global tiles and the window's
// band, or every past tile). Wave w owns query rows 16w..16w+15. Per key tile:
//   S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_16x16x32_bf16 (lane = query
//   row, 4 keys per 16-key subtile); dO is float32, so it enters as the sum
//   of three bf16 parts (an exact split), and every product is exact;
//   P = exp(S * scale - lse) on visible pairs, dS = P (dP - D) * scale with
//   D = rowsum(dO * O), formed in registers and written to LDS;
//   dQ += dS K on the same MFMA (dS as three bf16 parts, K read transposed
//   from an XOR-swizzled copy), kept in registers across key tiles;
//   dK = dS^T Q and dV = P^T dO in float32 FMAs from LDS (4 keys x 8 dims per
//   thread). The query tile's share of a key tile of the window's band goes
//   to a slot of its own in the workspace (plain stores) and
//   attn_bwd_reduce_kernel sums each key tile's slots; the share of a global
//   tile (seen by every query tile) and, without a workspace or in the dense
//   pattern, every share is added with one float atomic per element.
#include "common.h"
#include "internal.h"

typedef short v4i16 __attribute__((ext_vector_type(4)));

namespace sp {

constexpr int kBT = 64;         // rows per query tile, keys per key tile
constexpr int kBD = 128;        // head dim
constexpr int kBQs = kBD + 2;   // bf16 row stride of the Q tile read by the FMA phase (65 words: rows in distinct banks)
constexpr int kBKs = 136;       // bf16 row stride of the K and V tiles read as MFMA operands (272 B)
constexpr int kBPs = kBT + 1;   // float row stride of the P and dS tiles

struct BwdSmem {
  uint16_t q[kBT * kBQs];
  uint16_t ks[kBT * kBKs];
  uint16_t vs[kBT * kBKs];
  uint16_t kt[kBT * kBD];       // K row-major, 16-byte chunk c of row j at c ^ (j mod 16) (read transposed)
  float dO[kBT * (kBD + 1)];
  float P[kBT * kBPs];
  float dS[kBT * kBPs];
  float D[kBT], lse[kBT];
  uint32_t tiles[64];
};

// x = hi + mid + lo exactly: three round-to-nearest bf16 steps of a float32
// (each remainder is exact in float32 and has at most 16, then 8, bits left)
SP_DEV void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  const float r1 = x - bf16_to_f32(hi);
  mid = f32_to_bf16_rne(r1);
  lo = f32_to_bf16_rne(r1 - bf16_to_f32(mid));
}

__global__ __launch_bounds__(256) void attn_bwd_tile_kernel(AttnParams a, AttnBwd g) {
  __shared__ __attribute__((aligned(16))) BwdSmem sm;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qq = lane >> 4, c16 = lane & 15;
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
  const int gt = a.mode == 0 ? 0 : (min(a.n_global, L) + kBT - 1) / kBT;   // global tiles
  const int ntc = (a.ctx + kBT - 1) / kBT;
  if (a.mode == 0) {
    for (int t = tid; t <= last_tile; t += 256) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
  } else {
    const int wt = max(0, prow_first - a.window + 1) / kBT;
    for (int t = tid; t <= last_tile; t += 256)
      if (t < gt || t >= wt) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
  }
  __syncthreads();

  // ---- MFMA phases: lane column c16 = query row 16 wid + c16; the operand
  // dims of MFMA s are 32 qq + 8 s .. + 7 on both sides
  const int rloc = 16 * wid + c16;
  const bool rvalid = rloc < nrows;
  const int prow = pbase + q0 + rloc;
  const float lr = sm.lse[rloc], Dr = sm.D[rloc];
  bf16x8 Qb[4];
  u32x4 Ob[3][4];                  // the row's dO as three bf16 parts
  if (rvalid) {
    const uint16_t* qp = (const uint16_t*)a.q.p + b * a.q.s[0] + h * a.q.s[1] + (int64_t)(q0 + rloc) * a.q.s[2] + 32 * qq;
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s] = *(const bf16x8*)(qp + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s] = (bf16x8){};
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* dr = &sm.dO[rloc * (kBD + 1) + 32 * qq + 8 * s + 2 * u];   // zero rows past nrows
      uint32_t h0, m0, l0, h1, m1, l1;
      split3(dr[0], h0, m0, l0);
      split3(dr[1], h1, m1, l1);
      Ob[0][s][u] = h0 | (h1 << 16);
      Ob[1][s][u] = m0 | (m1 << 16);
      Ob[2][s][u] = l0 | (l1 << 16);
    }
  f32x4 dQ[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) dQ[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // FMA phase mapping: keys orow.., dims odim..
  const int orow = 4 * (tid >> 4), odim = 8 * (tid & 15);
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
      // stage K (row-major and swizzled) and V (keys past L read as row L-1, masked below)
      for (int e = tid; e < kBT * kBD / 8; e += 256) {
        const int key = e >> 4, col = e & 15;
        const int j = min(j0 + key, L - 1);
        const u32x4 kv = *(const u32x4*)(kbase + (int64_t)j * a.k.s[2] + 8 * col);
        const u32x4 vv = *(const u32x4*)(vbase + (int64_t)j * a.v.s[2] + 8 * col);
        *(u32x4*)&sm.ks[key * kBKs + 8 * col] = kv;
        *(u32x4*)&sm.kt[key * kBD + 8 * (col ^ (key & 15))] = kv;
        *(u32x4*)&sm.vs[key * kBKs + 8 * col] = vv;
      }
      __syncthreads();
      // S^T and dP^T: lane holds row rloc, keys 16 st + 4 qq + v
      f32x4 S[4], dP[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        S[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
        dP[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const uint16_t* kr = &sm.ks[(16 * st + c16) * kBKs + 32 * qq];
        const uint16_t* vr = &sm.vs[(16 * st + c16) * kBKs + 32 * qq];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kr + 8 * s), Qb[s], S[st], 0, 0, 0);
          const bf16x8 vA = *(const bf16x8*)(vr + 8 * s);
#pragma unroll
          for (int pt = 0; pt < 3; ++pt)
            dP[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, *(const bf16x8*)&Ob[pt][s], dP[st], 0, 0, 0);
        }
      }
      // P and dS on visible pairs (registers for dQ, LDS for dK and dV)
      float dz[16];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int kl = 16 * st + 4 * qq + v;
          const int j = j0 + kl;
          bool vis = rvalid && j <= prow && lr > -INFINITY;
          if (vis && a.mode == 2) vis = j >= prow - a.window + 1 || j < a.n_global;
          const float p = vis ? expf(S[st][v] * a.scale - lr) : 0.f;
          const float ds = p * (dP[st][v] - Dr) * a.scale;
          dz[4 * st + v] = ds;
          sm.P[rloc * kBPs + kl] = p;
          sm.dS[rloc * kBPs + kl] = ds;
        }
      // dQ += dS K: A = dS (three parts), k = 8 qq + v <-> keys 4 qq + v (v < 4), 16 + 4 qq + (v - 4),
      // in two halves of 32 keys; B = K^T by transposed reads of the swizzled copy
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 A0, A1, A2;
#pragma unroll
        for (int v2 = 0; v2 < 4; ++v2) {
          const int i0 = (v2 < 2) ? (8 * hf + 2 * v2) : (8 * hf + 4 + 2 * (v2 - 2));
          uint32_t h0, m0, l0, h1, m1, l1;
          split3(dz[i0], h0, m0, l0);
          split3(dz[i0 + 1], h1, m1, l1);
          A0[v2] = h0 | (h1 << 16);
          A1[v2] = m0 | (m1 << 16);
          A2[v2] = l0 | (l1 << 16);
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const int tr0 = 32 * hf + 4 * qq + (c16 >> 2), tr1 = tr0 + 16;
          const int lch = 2 * nt + ((4 * (c16 & 3)) >> 3), wth = (4 * (c16 & 3)) & 7;
          const v4i16 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)&sm.kt[tr0 * kBD + 8 * (lch ^ (tr0 & 15)) + wth]);
          const v4i16 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)&sm.kt[tr1 * kBD + 8 * (lch ^ (tr1 & 15)) + wth]);
          u32x4 Bk;
          Bk[0] = (uint32_t)(uint16_t)b0[0] | ((uint32_t)(uint16_t)b0[1] << 16);
          Bk[1] = (uint32_t)(uint16_t)b0[2] | ((uint32_t)(uint16_t)b0[3] << 16);
          Bk[2] = (uint32_t)(uint16_t)b1[0] | ((uint32_t)(uint16_t)b1[1] << 16);
          Bk[3] = (uint32_t)(uint16_t)b1[2] | ((uint32_t)(uint16_t)b1[3] << 16);
          dQ[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&A0, *(const bf16x8*)&Bk, dQ[nt], 0, 0, 0);
          dQ[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&A1, *(const bf16x8*)&Bk, dQ[nt], 0, 0, 0);
          dQ[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&A2, *(const bf16x8*)&Bk, dQ[nt], 0, 0, 0);
        }
      }
      __syncthreads();
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
      if (g.part && t >= gt) {
        // band tile: this query tile's share into its slot ([key][dim] dK,
        // then dV); the query tiles that see a band key tile are
        // consecutive and at most nslot of them, so qt mod nslot tells
        // them apart
        const int slot = qt % g.nslot;
        float* pp = g.part + ((((int64_t)b * a.Hq + h) * ntc + t) * g.nslot + slot) * (kBT * kBD * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* pk = pp + (orow + i) * kBD + odim;
          *(f32x4*)pk = (f32x4){dk[i][0], dk[i][1], dk[i][2], dk[i][3]};
          *(f32x4*)(pk + 4) = (f32x4){dk[i][4], dk[i][5], dk[i][6], dk[i][7]};
          *(f32x4*)(pk + kBT * kBD) = (f32x4){dv[i][0], dv[i][1], dv[i][2], dv[i][3]};
          *(f32x4*)(pk + kBT * kBD + 4) = (f32x4){dv[i][4], dv[i][5], dv[i][6], dv[i][7]};
        }
      } else {
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
      }
      __syncthreads();
    }
  }
  // ---- dQ: lane holds dims 16 nt + c16 of rows 16 wid + 4 qq + v
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = 16 * wid + 4 * qq + v;
    if (rr >= nrows) continue;
    float* dqr = g.dq + b * g.dqs[0] + h * g.dqs[1] + (int64_t)(q0 + rr) * g.dqs[2];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) dqr[16 * nt + c16] = dQ[nt][v];
  }
}

// Sums the slots of one band key tile: workgroup (t, quarter) x (KV head,
// request) takes 16 keys x 128 dims of dK and dV; the (query head, query
// tile) pairs that wrote a slot for tile t follow from the same tile sets as
// in the tile kernel and are listed in LDS, then read four at a time with
// every load of a batch in flight together.
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(AttnParams a, AttnBwd g) {
  __shared__ uint32_t lst[1024];
  __shared__ uint32_t nl;
  const int t = blockIdx.x >> 2, quarter = blockIdx.x & 3, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int ntiles_all = (L + kBT - 1) / kBT;
  const int gt = (min(a.n_global, L) + kBT - 1) / kBT;
  if (t < gt) return;   // global tiles: float atomics onto rows zeroed before the tile kernel
  const int pbase = L - a.Nq, nqt = (a.Nq + kBT - 1) / kBT, G = a.Hq / a.Hkv;
  const int ntc = (a.ctx + kBT - 1) / kBT;
  if (tid == 0) nl = 0u;
  __syncthreads();
  for (int e = tid; t < ntiles_all && e < G * nqt; e += 256) {
    const int hq = kvh * G + e / nqt, qt = e % nqt;
    const int q0 = qt * kBT, nrows = min(kBT, a.Nq - q0);
    const int prow_first = pbase + q0, prow_last = prow_first + nrows - 1;
    const int last_tile = min(ntiles_all - 1, prow_last / kBT);
    const int wt = max(0, prow_first - a.window + 1) / kBT;
    const int slot = qt % g.nslot;
    if (prow_last >= 0 && t >= wt && t <= last_tile) {
      const uint32_t x = atomicAdd(&nl, 1u);
      if (x < 1024u) lst[x] = (uint32_t)(((hq * ntc + t) * g.nslot + slot));
    }
  }
  __syncthreads();
  // a tile past the context or seen by no query tile has no slots: its rows
  // are written as zeros
  const int n = (int)min(nl, 1024u);
  // thread: key 16 quarter + tid / 16, dims 8 (tid % 16) .. +7 of dK and of dV
  const int kr = 16 * quarter + (tid >> 4), dd = 8 * (tid & 15);
  const int64_t base = (int64_t)b * a.Hq * ntc * g.nslot;
  f32x4 ak0 = {0.f, 0.f, 0.f, 0.f}, ak1 = ak0, av0 = ak0, av1 = ak0;
  for (int i = 0; i < n; i += 4) {
    f32x4 x[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* pp = g.part + (base + lst[min(i + u, n - 1)]) * (kBT * kBD * 2) + kr * kBD + dd;
      x[u][0] = *(const f32x4*)pp;
      x[u][1] = *(const f32x4*)(pp + 4);
      x[u][2] = *(const f32x4*)(pp + kBT * kBD);
      x[u][3] = *(const f32x4*)(pp + kBT * kBD + 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wu = i + u < n ? 1.f : 0.f;   // past the list: loaded again, weight 0
      ak0 += x[u][0] * wu;
      ak1 += x[u][1] * wu;
      av0 += x[u][2] * wu;
      av1 += x[u][3] * wu;
    }
  }
  const int j = t * kBT + kr;
  if (j >= a.ctx) return;   // rows L .. ctx - 1 get zeros (no query sees them)
  float* dkr = g.dk + b * g.dks[0] + kvh * g.dks[1] + (int64_t)j * g.dks[2] + dd;
  float* dvr = g.dv + b * g.dvs[0] + kvh * g.dvs[1] + (int64_t)j * g.dvs[2] + dd;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dkr[e] = ak0[e];
    dkr[4 + e] = ak1[e];
    dvr[e] = av0[e];
    dvr[4 + e] = av1[e];
  }
}

// rows of dK/dV to zero before the backward: with workspace slots only the
// global tiles' rows (the reduce kernel writes every other row, zeros
// included), otherwise every row
int attn_bwd_zero_rows(const AttnParams& a, const AttnBwd& g) {
  if (!(attn_bwd_tile_ok(a) && g.part && attn_bwd_slots(a) > 0)) return a.ctx;
  return min(a.ctx, (a.n_global + kBT - 1) / kBT * kBT);
}

// slots per band key tile: the query tiles that see a band key tile t have
// their first positions P0 (64 apart) in [64 t - 63, 64 t + 62 + window],
// so there are at most floor((125 + window) / 64) + 1 <= window / 64 + 3 of
// them, consecutive (a query tile need not start on a key tile, and the
// last one may be short)
int attn_bwd_slots(const AttnParams& a) { return a.mode == 2 && a.stride == 0 ? a.window / kBT + 3 : 0; }

bool attn_bwd_tile_ok(const AttnParams& a) {
  return a.q.dt == DT_BF16 && a.d == kBD && !a.ptab && (a.mode == 0 || (a.mode == 2 && a.stride == 0)) &&
         (a.ctx + kBT - 1) / kBT <= 2048;
}

hipError_t launch_attn_bwd_tile(const AttnParams& a, const AttnBwd& g, hipStream_t st) {
  dim3 grid((a.Nq + kBT - 1) / kBT, a.Hq, a.B);
  hipLaunchKernelGGL(attn_bwd_tile_kernel, grid, dim3(256), 0, st, a, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !g.part) return e;
  hipLaunchKernelGGL(attn_bwd_reduce_kernel, dim3(4 * ((a.ctx + kBT - 1) / kBT), a.Hkv, a.B), dim3(256), 0, st, a, g);
  return hipGetLastError();
}

}  // namespace sp
