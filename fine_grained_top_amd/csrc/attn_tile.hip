// Tiled sparse attention for fixed visible sets (dense causal, sliding window
// + global tokens, selected blocks + window), bf16, d = 128.
//
// One workgroup = 64 query rows of one (request, head); wave w owns rows
// 16w..16w+15. Key tiles of 64 keys are visited in increasing order: the
// global tiles and the band of the window (WINDOW_GLOBAL), every past tile
// (DENSE), or the union of the rows' selected blocks and windows (BLOCKS,
// from an LDS tile bitmap). A dilated stride adds tiles of 64 consecutive
// multiples of the stride (K/V rows read at that stride), masked to the keys
// outside each row's window and global prefix, which the first stream covers. K and V tiles are staged row-major in LDS (V
// with XOR-swizzled 16-byte chunks, read as the MFMA operand by transposed
// LDS reads); the next tile is prefetched into registers while the current
// one is consumed. Per wave and tile: S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (lane = query row, 4 keys per 16-key subtile),
// per-element masks from the row's visible set, online softmax in float32
// (exp2), and O += P V with P as a bf16 hi/lo pair. In BLOCKS mode a wave
// skips a tile no row of its own can see.
#include "common.h"
#include "internal.h"

typedef short v4i16 __attribute__((ext_vector_type(4)));

namespace sp {

constexpr int kTQ = 64, kTK = 64;
constexpr int kKs = 136;       // K tile row stride in 16-bit words (272 B)
constexpr int kMaxBlkWords = 64;   // per-row block bitmap words (<= 2048 blocks)
constexpr float kLog2eT = 1.4426950408889634f;
constexpr float kLn2T = 0.6931471805599453f;

// Every tile array starts on a 16-byte boundary (16-byte LDS stores, 8-byte
// transposed reads), whatever the sizes of the arrays before it.
template <bool SPLIT, bool BLK>
struct TileSmem {
  alignas(16) uint16_t ks[kTK * kKs];
  alignas(16) uint16_t vt[64 * 128];    // V tile row-major, XOR-swizzled 16-byte chunks
  uint32_t tiles[64];                    // tile bitmap (<= 2048 tiles)
  uint32_t rowblk[BLK ? kTQ * kMaxBlkWords : 1];   // BLOCKS: per-row selected-block bitmaps
  alignas(16) uint16_t ks2[SPLIT ? kTK * kKs : 8];   // SPLIT: the low parts, laid out as ks / vt
  alignas(16) uint16_t vt2[SPLIT ? 64 * 128 : 8];
};
using TileSmemSplit = TileSmem<true, false>;
using TileSmemSplitBlk = TileSmem<true, true>;
static_assert(__builtin_offsetof(TileSmemSplit, ks2) % 16 == 0 && __builtin_offsetof(TileSmemSplit, vt2) % 16 == 0 &&
                  __builtin_offsetof(TileSmemSplitBlk, ks2) % 16 == 0,
              "tile arrays on 16-byte boundaries");

// STRIDE: window/global mode with a dilated stride (the second key stream).
// SPLIT: compressed entries held as two bf16 parts (hi in k/v, lo in
// klo/vlo): S = K_hi Q^T + K_lo Q^T and O += P V_hi + P_hi V_lo (the term
// P_lo V_lo is below 2^-16 of the product), so the entries keep ~16
// significant bits instead of bf16's 8.
// MODE: the selection mode, fixed per instance so that the per-element masks
// carry no tests of other modes.
// Three waves per SIMD (at most 168 VGPRs, no spills) and, outside BLOCKS
// mode, no per-row block bitmaps in LDS (34 KB): three workgroups per CU.
template <int MODE, bool STRIDE, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_tile_kernel(AttnParams a, int xper) {
  __shared__ __attribute__((aligned(16))) TileSmem<SPLIT, MODE == 3> sm;
  // query tiles of a head are consecutive items, and each XCD takes a run of
  // them: the key tiles that neighbouring query tiles share stay in its L2
  const int nqt = (a.Nq + kTQ - 1) / kTQ;
  const int item = xcd_item(blockIdx.x, xper);
  if (item >= nqt * a.Hq * a.B) return;
  const int qt = item % nqt, h = (item / nqt) % a.Hq, b = item / (nqt * a.Hq);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qq = lane >> 4, c16 = lane & 15;
  const int kvh = h / (a.Hq / a.Hkv);
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int q0 = qt * kTQ;
  const int pbase = L - a.Nq;                      // position of row 0
  const int prow_first = pbase + q0;
  const int prow_last = pbase + min(q0 + kTQ, a.Nq) - 1;
  // mode 5 (compressed entries): key rows are the request's complete blocks,
  // entry c visible at position p when c <= (p + 1) / bs - 1
  const int Lk = MODE == 5 ? L / a.bs : L;
  const int ntiles_all = (Lk + kTK - 1) / kTK;
  const int nbk = MODE == 3 ? (a.ctx + a.bs - 1) / a.bs : 0;
  const int bwords = (nbk + 31) >> 5;

  // ---- tile set of this query tile
  for (int i = tid; i < 64; i += 256) sm.tiles[i] = 0;
  if (MODE == 3)
    for (int i = tid; i < kTQ * bwords; i += 256) sm.rowblk[i] = 0;
  __syncthreads();
  const int plast_v = MODE == 5 ? (prow_last + 1) / a.bs - 1 : prow_last;
  const int last_tile = plast_v >= 0 ? min(ntiles_all - 1, plast_v / kTK) : -1;
  // dilated stride: multiples m * stride, m in [m_lo, m_hi], below the latest
  // window start of the tile and outside the global prefix, as nvt virtual
  // tiles numbered from ntiles_all
  const int NT = ntiles_all;
  const int sd = STRIDE ? a.stride : 0;
  int m_lo = 0, nvt = 0;
  if (STRIDE && prow_last - a.window >= 0) {
    m_lo = (a.n_global + sd - 1) / sd;
    const int m_hi = (prow_last - a.window) / sd;
    if (m_hi >= m_lo) nvt = (m_hi - m_lo + kTK) / kTK;
  }
  if (MODE == 0 || MODE == 5) {
    for (int t = tid; t <= last_tile; t += 256) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
  } else if (MODE == 2) {
    const int gt = (min(a.n_global, L) + kTK - 1) / kTK;
    const int wt = max(0, prow_first - a.window + 1) / kTK;
    for (int t = tid; t <= last_tile; t += 256)
      if (t < gt || t >= wt) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
  } else {
    const int wt = max(0, prow_first - a.window + 1) / kTK;
    for (int t = wt + tid; t <= last_tile; t += 256) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
    for (int e = tid; e < kTQ * a.K; e += 256) {
      const int rr = e / a.K, slot = e % a.K;
      if (q0 + rr >= a.Nq) continue;
      const int blk = a.sel[b * a.sels[0] + (h / (a.Hq / a.G_sel)) * a.sels[1] + (int64_t)(q0 + rr) * a.sels[2] + slot];
      if (blk < 0 || blk >= nbk) continue;
      atomicOr(&sm.rowblk[rr * bwords + (blk >> 5)], 1u << (blk & 31));
      const int t0 = (blk * a.bs) / kTK, t1 = min(ntiles_all - 1, (blk * a.bs + a.bs - 1) / kTK);
      for (int t = t0; t <= t1; ++t) atomicOr(&sm.tiles[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();

  // ---- per-lane row state: lane column c16 = query row 16*wid + c16
  const int rloc = 16 * wid + c16;
  const int rq = q0 + rloc;
  const bool rvalid = rq < a.Nq;
  const int prow = pbase + rq;
  const int prow_v = MODE == 5 ? (prow + 1) / a.bs - 1 : prow;   // last visible key row
  const int wstart = prow - a.window + 1;
  bf16x8 Qb[4];
  if (rvalid) {
    const uint16_t* qp = (const uint16_t*)a.q.p + b * a.q.s[0] + h * a.q.s[1] + (int64_t)rq * a.q.s[2] + 32 * qq;
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s] = *(const bf16x8*)(qp + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s] = (bf16x8){};
  }
  const float cs = a.scale * kLog2eT;
  float m = -INFINITY, l = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.s[0] + kvh * a.k.s[1];
  const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.s[0] + kvh * a.v.s[1];
  const uint16_t* kbase2 = SPLIT ? (const uint16_t*)a.klo + b * a.k.s[0] + kvh * a.k.s[1] : nullptr;
  const uint16_t* vbase2 = SPLIT ? (const uint16_t*)a.vlo + b * a.v.s[0] + kvh * a.v.s[1] : nullptr;

  // next tile after t (or -1)
  auto next_tile = [&](int t) -> int {
    for (int w = (t + 1) >> 5; w <= (last_tile >> 5) && w < 64; ++w) {
      uint32_t bits = sm.tiles[w];
      if (w == ((t + 1) >> 5)) bits &= ~0u << ((t + 1) & 31);
      if (bits) {
        const int nt = w * 32 + __builtin_ctz(bits);
        return nt <= last_tile ? nt : -1;
      }
    }
    return -1;
  };
  // next tile of either stream
  auto next_any = [&](int t) -> int {
    if (STRIDE && t >= NT) return t + 1 < NT + nvt ? t + 1 : -1;
    const int n = t < last_tile ? next_tile(t) : -1;
    return n >= 0 ? n : (STRIDE && nvt > 0 ? NT : -1);
  };
  // prefetch of one tile: chunk c = tid + 256u -> key c/16, 16-byte column c%16
  u32x4 pk[4], pv[4];
  u32x4 pk2[SPLIT ? 4 : 1], pv2[SPLIT ? 4 : 1];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      int j = (!STRIDE || t < NT) ? t * kTK + (c >> 4) : (m_lo + (t - NT) * kTK + (c >> 4)) * sd;
      j = j < Lk ? j : Lk - 1;
      pk[u] = *(const u32x4*)(kbase + (int64_t)j * a.k.s[2] + 8 * (c & 15));
      pv[u] = *(const u32x4*)(vbase + (int64_t)j * a.v.s[2] + 8 * (c & 15));
      if constexpr (SPLIT) {
        pk2[u] = *(const u32x4*)(kbase2 + (int64_t)j * a.k.s[2] + 8 * (c & 15));
        pv2[u] = *(const u32x4*)(vbase2 + (int64_t)j * a.v.s[2] + 8 * (c & 15));
      }
    }
  };
  int t = next_any(-1);
  if (t >= 0) load_tile(t);
  while (t >= 0) {
    // stage the prefetched tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int key = c >> 4, col = c & 15;
      *(u32x4*)&sm.ks[key * kKs + 8 * col] = pk[u];
      // V row-major, 16-byte chunk col of row key at col ^ (key mod 16)
      *(u32x4*)&sm.vt[key * 128 + 8 * (col ^ (key & 15))] = pv[u];
      if constexpr (SPLIT) {
        *(u32x4*)&sm.ks2[key * kKs + 8 * col] = pk2[u];
        *(u32x4*)&sm.vt2[key * 128 + 8 * (col ^ (key & 15))] = pv2[u];
      }
    }
    __syncthreads();
    const int tn = next_any(t);
    if (tn >= 0) load_tile(tn);

    const bool sv = STRIDE && t >= NT;             // a tile of stride multiples
    const int j0 = sv ? 0 : t * kTK;
    const int mb0 = sv ? m_lo + (t - NT) * kTK : 0;
    // does any row of this wave see this tile?
    bool see = rvalid && prow_v >= j0;
    if (sv) see = rvalid && mb0 * sd <= prow && mb0 * sd < wstart;
    else if (see && MODE == 2) see = (j0 + kTK - 1 >= wstart) || (j0 < a.n_global);
    if (see && MODE == 3) {
      bool any = j0 + kTK - 1 >= wstart;
      if (!any) {
        const int b0 = j0 / a.bs, b1 = min(nbk - 1, (j0 + kTK - 1) / a.bs);
        for (int bb = b0; bb <= b1 && !any; ++bb)
          any = (sm.rowblk[rloc * bwords + (bb >> 5)] >> (bb & 31)) & 1u;
      }
      see = any;
    }
    if (__ballot(see)) {
      // S^T for the 4 subtiles of 16 keys: lane holds row c16, keys 16*st + 4*qq + v
      f32x4 S[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        S[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const uint16_t* kr = &sm.ks[(16 * st + c16) * kKs + 32 * qq];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kr + 8 * s), Qb[s], S[st], 0, 0, 0);
        if constexpr (SPLIT) {
          const uint16_t* kr2 = &sm.ks2[(16 * st + c16) * kKs + 32 * qq];
#pragma unroll
          for (int s = 0; s < 4; ++s)
            S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kr2 + 8 * s), Qb[s], S[st], 0, 0, 0);
        }
      }
      // masks: lane's keys j = j0 + 16*st + 4*qq + v for its row (column c16);
      // in a stride tile the keys are multiples (mb0 + 16*st + 4*qq + v) * stride
      float z[16];
      float tm = -INFINITY;
      if (!sv) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int j = j0 + 16 * st + 4 * qq + v;
            bool vis = rvalid && j <= prow_v;
            if (vis && MODE == 2) vis = j >= wstart || j < a.n_global;
            if (vis && MODE == 3) {
              const int bb = j / a.bs;
              vis = j >= wstart || ((sm.rowblk[rloc * bwords + (bb >> 5)] >> (bb & 31)) & 1u);
            }
            const float zz = vis ? S[st][v] * cs : -INFINITY;
            z[4 * st + v] = zz;
            tm = fmaxf(tm, zz);
          }
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int j = (mb0 + 16 * st + 4 * qq + v) * sd;
            const bool vis = rvalid && j <= prow && j < wstart && j >= a.n_global;
            const float zz = vis ? S[st][v] * cs : -INFINITY;
            z[4 * st + v] = zz;
            tm = fmaxf(tm, zz);
          }
      }
      tm = rows4_max(tm);
      const float mn = fmaxf(m, tm);
      // lazy rescale: P is formed against the reference maximum m, which
      // moves (rescaling O and l) only when some row's maximum has grown past
      // it by more than 8 (log2 units), so P stays below 2^8 (exact in the
      // bf16 hi/lo pair, far from float32 overflow); the branch is the same
      // for the whole wave and rarely taken after the first tiles. The split
      // compressed-entry instance keeps the per-tile rescale: the lazy form
      // costs it registers and an occupancy step.
      constexpr bool kLazy = !(MODE == 5 && SPLIT);
      const bool up = kLazy ? __any(mn > m + 8.f) : true;
      const float mr = up ? mn : m;
      float alpha = 1.f, ps = 0.f;
      if (mr > -INFINITY) {
        if (up) alpha = exp2f(m - mr);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          z[i] = exp2f(z[i] - mr);
          ps += z[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
      }
      ps = rows4_sum(ps);
      l = l * alpha + ps;
      m = mr;
#pragma unroll
      for (int v = 0; v < 4 && up; ++v) {
        // alpha of row r lives in lane r: four readlanes, picked by the lane's row group
        const int ai = __builtin_bit_cast(int, alpha);
        const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, v));
        const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 4 + v));
        const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 8 + v));
        const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 12 + v));
        const float av = qq == 0 ? a0 : qq == 1 ? a1 : qq == 2 ? a2 : a3;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) O[nt][v] *= av;
      }
      // O += P V, two halves of 32 keys; k = 8*qq + v <-> keys 4*qq+v (v<4), 16+4*qq+(v-4)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 Ahi, Alo;
#pragma unroll
        for (int v2 = 0; v2 < 4; ++v2) {
          const int i0 = (v2 < 2) ? (8 * hf + 2 * v2) : (8 * hf + 4 + 2 * (v2 - 2));
          const float x0 = z[i0], x1 = z[i0 + 1];
          const uint32_t h0b = f32_to_bf16_rne(x0), h1b = f32_to_bf16_rne(x1);
          Ahi[v2] = h0b | (h1b << 16);
          Alo[v2] = f32_to_bf16_rne(x0 - bf16_to_f32(h0b)) | (f32_to_bf16_rne(x1 - bf16_to_f32(h1b)) << 16);
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          // B operand by two LDS transposed reads: lane (qq, j) points at key
          // row 32 hf + 4 qq + j / 4 (+16), dims 16 nt + 4 (j mod 4) .. +3, and
          // receives dim 16 nt + j of its group's four rows
          const int tr0 = 32 * hf + 4 * qq + (c16 >> 2), tr1 = tr0 + 16;
          const int lch = 2 * nt + ((4 * (c16 & 3)) >> 3), wth = (4 * (c16 & 3)) & 7;
          const v4i16 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)&sm.vt[tr0 * 128 + 8 * (lch ^ (tr0 & 15)) + wth]);
          const v4i16 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)&sm.vt[tr1 * 128 + 8 * (lch ^ (tr1 & 15)) + wth]);
          u32x4 Bv;
          Bv[0] = (uint32_t)(uint16_t)a0[0] | ((uint32_t)(uint16_t)a0[1] << 16);
          Bv[1] = (uint32_t)(uint16_t)a0[2] | ((uint32_t)(uint16_t)a0[3] << 16);
          Bv[2] = (uint32_t)(uint16_t)a1[0] | ((uint32_t)(uint16_t)a1[1] << 16);
          Bv[3] = (uint32_t)(uint16_t)a1[2] | ((uint32_t)(uint16_t)a1[3] << 16);
          O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&Ahi, *(const bf16x8*)&Bv, O[nt], 0, 0, 0);
          O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&Alo, *(const bf16x8*)&Bv, O[nt], 0, 0, 0);
          if constexpr (SPLIT) {
            const v4i16 c0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)&sm.vt2[tr0 * 128 + 8 * (lch ^ (tr0 & 15)) + wth]);
            const v4i16 c1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)&sm.vt2[tr1 * 128 + 8 * (lch ^ (tr1 & 15)) + wth]);
            u32x4 B2;
            B2[0] = (uint32_t)(uint16_t)c0[0] | ((uint32_t)(uint16_t)c0[1] << 16);
            B2[1] = (uint32_t)(uint16_t)c0[2] | ((uint32_t)(uint16_t)c0[3] << 16);
            B2[2] = (uint32_t)(uint16_t)c1[0] | ((uint32_t)(uint16_t)c1[1] << 16);
            B2[3] = (uint32_t)(uint16_t)c1[2] | ((uint32_t)(uint16_t)c1[3] << 16);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&Ahi, *(const bf16x8*)&B2, O[nt], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
    t = tn;
  }

  // ---- normalize and write: lane holds dims 16*nt + c16 of rows 4*qq + v (of this wave)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = 16 * wid + 4 * qq + v;
    const float lr = __shfl(l, 4 * qq + v, 64);
    const float mr = __shfl(m, 4 * qq + v, 64);
    if (q0 + rr >= a.Nq) continue;
    float* o = a.o + b * a.os[0] + h * a.os[1] + (int64_t)(q0 + rr) * a.os[2];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[16 * nt + c16] = O[nt][v] * inv;
    if (a.lse && c16 == 0)
      a.lse[((int64_t)b * a.Hq + h) * a.Nq + q0 + rr] = lr > 0.f ? (mr + log2f(lr)) * kLn2T : -INFINITY;
  }
}

bool attn_tile_ok(const AttnParams& a) {
  if (a.q.dt != DT_BF16 || a.d != 128 || a.mode == 1 || a.mode == 4 || a.ptab) return false;
  if ((a.ctx + kTK - 1) / kTK > 2048) return false;
  if (a.mode == 3 && ((a.ctx + a.bs - 1) / a.bs > 32 * kMaxBlkWords)) return false;
  return true;
}

hipError_t launch_attn_tile(const AttnParams& a, hipStream_t st) {
  const int items = (a.Nq + kTQ - 1) / kTQ * a.Hq * a.B;
  const int per = (items + 7) / 8;
  const dim3 grid(8 * per);
  if (a.mode == 2 && a.stride > 0) hipLaunchKernelGGL((attn_tile_kernel<2, true, false>), grid, dim3(256), 0, st, a, per);
  else if (a.mode == 2) hipLaunchKernelGGL((attn_tile_kernel<2, false, false>), grid, dim3(256), 0, st, a, per);
  else if (a.mode == 5 && a.klo) hipLaunchKernelGGL((attn_tile_kernel<5, false, true>), grid, dim3(256), 0, st, a, per);
  else if (a.mode == 5) hipLaunchKernelGGL((attn_tile_kernel<5, false, false>), grid, dim3(256), 0, st, a, per);
  else if (a.mode == 3) hipLaunchKernelGGL((attn_tile_kernel<3, false, false>), grid, dim3(256), 0, st, a, per);
  else hipLaunchKernelGGL((attn_tile_kernel<0, false, false>), grid, dim3(256), 0, st, a, per);
  return hipGetLastError();
}

}  // namespace sp
