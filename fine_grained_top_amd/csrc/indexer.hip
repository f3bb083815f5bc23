// Indexer scores: s(i,j) = q_I[i] . k_I[j]  or  sum_h w_h * max(0, q_I[i,h] . k_I[j]).
//
// Two kernels:
//  * idx_mfma64: d_I = 64, bf16 queries, bf16 or fp8-e4m3 keys, one key head
//    shared by every selection group, at most 128 (query row, head) slots per
//    request (decode and short prefill). Keys stream from HBM once; each wave
//    turns 32 keys into a 32x32x16 bf16 MFMA B operand (fp8 upconverted to
//    bf16 exactly) against the resident query slots, and reduces the heads
//    of a group in-lane in the epilogue.
//    With page keys requested (pages of 32..512 keys), the epilogue also
//    folds each tile's scores per selection row (DPP rotations inside 16-lane
//    rows and a row swap give the maximum over the half-wave's 32 keys) and
//    merges them per page in LDS: the largest score of every (row, page).
//  * idx_generic: any supported dtype/shape, one key per thread, FMA chain.
// Both record, per 512/256-key chunk, the largest |k| element, from which
// idx_err derives each row's rigorous bound |score - key|.
#include "common.h"
#include "internal.h"

namespace sp {

constexpr int kMfmaChunk = 512;   // keys per workgroup in idx_mfma64
constexpr int kGenChunk = 256;    // keys per workgroup in idx_generic

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

SP_DEV float load_val(const void* p, int dt, int64_t i) {
  if (dt == DT_F32) return ((const float*)p)[i];
  if (dt == DT_BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  return fp8_to_f32(((const uint8_t*)p)[i]);
}

// ----------------------------------------------------------------------------
// MODE: 0 scores, 1 threshold filter (candidate lists), 2 scores and page keys.
// CPW: consecutive 512-key chunks per workgroup (one request); PD: tiles of
// 32 keys each wave keeps in flight. Each wave walks its CPW * 4 tiles in
// order, the key bytes of tile t + PD requested as tile t is scored, so the
// loads of a workgroup stream while it computes (PD = CPW * 4: all at once).
// RL (filter, one selection group): survivors go to per-row lists, staged in
// LDS per (row, wave) and moved out by each wave on its own (one global
// reservation per row with entries) when a region could overflow, and at the
// wave's end.
template <int KT, int NMB, int HPG, bool RELU, int MODE, int CPW, int PD, bool RL = false>
__global__ __launch_bounds__(256) void idx_mfma64_kernel(IndexerParams p) {
  constexpr bool FILTER = MODE == 1;
  constexpr bool PM = MODE == 2;
  constexpr int TPW = kMfmaChunk / 32 / 4;   // tiles per wave and chunk
  constexpr int NT = CPW * TPW;              // tiles per wave
  constexpr int RW = KT == DT_FP8 ? 2 : 4;   // 16-byte loads per lane and tile
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int jw = blockIdx.x * CPW * kMfmaChunk;        // first key of the workgroup
  if (jw >= L) return;
  const int M = p.Nq * p.H_I;
  const int hshift = __builtin_ctz(p.H_I);
  const int mbase = 128 * blockIdx.z;                 // first (row, head) slot of this workgroup
  // causal skip: no row of this slot block sees any key of the chunks
  {
    const int rmax = min(p.Nq - 1, (mbase + 32 * NMB - 1) >> hshift);
    if (jw > L - p.Nq + rmax) return;
  }
  // key bytes of tile t: key jw + (t / 4) * 512 + (wid + 4 (t % 4)) * 32 + col,
  // dims 32 half .. 32 half + 31
  auto tile_key = [&](int t) { return jw + (t / TPW) * kMfmaChunk + (wid + 4 * (t % TPW)) * 32 + col; };
  auto load = [&](int t, u32x4 (&dst)[RW]) {
    const int j = tile_key(t);
    const int jc = j < L ? j : L - 1;
    if (KT == DT_FP8) {
      const uint8_t* kp = (const uint8_t*)p.k.p + b * p.k.s[0] + (int64_t)jc * p.k.s[1] + 32 * half;
      dst[0] = *(const u32x4*)kp;
      dst[1] = *(const u32x4*)(kp + 16);
    } else {
      const uint16_t* kp = (const uint16_t*)p.k.p + b * p.k.s[0] + (int64_t)jc * p.k.s[1] + 32 * half;
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c] = *(const u32x4*)(kp + 8 * c);
    }
  };
  u32x4 raw[PD][RW];
#pragma unroll
  for (int t = 0; t < PD && t < NT; ++t) load(t, raw[t]);

  // A operands: query slot m = mbase + 32*mb + col, dims 32*half + 8*s + v (s = k-step)
  bf16x8 A[NMB][4];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int m = mbase + 32 * mb + col;
    if (m < M) {
      const int r = m >> hshift, h = m & (p.H_I - 1);
      const uint16_t* qp = (const uint16_t*)p.q.p + b * p.q.s[0] + r * p.q.s[1] + h * p.q.s[2] + 32 * half;
#pragma unroll
      for (int s = 0; s < 4; ++s) A[mb][s] = *(const bf16x8*)(qp + 8 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) A[mb][s] = (bf16x8){};
    }
  }

  __shared__ uint32_t lcount[FILTER ? CPW : 1][128];
  // RL: every (row, wave) pair owns a stage region of two tiles' keys (a
  // tile adds at most 32 entries to it); the wave counts its entries of each
  // row in scalar registers (no LDS atomics), writes every lane's candidate
  // unconditionally (lanes that fail the threshold into a discard slot of
  // their own), and moves its stage to the rows' lists by itself (one global
  // reservation per row, no workgroup barrier) when a region could overflow
  // on the next tile, and once at its end
  constexpr int kRlRows = 128 / HPG;                  // rows of a 128-slot block (one group per row)
  constexpr int kRlSlots = 64;                        // stage entries per (row, wave)
  constexpr int kRlDiscard = kRlRows * 4 * kRlSlots;  // first discard slot
  __shared__ u32x2 stage[RL ? kRlDiscard + 256 : 1];
  __shared__ uint32_t wpre[RL ? 4 : 1][RL ? kRlRows + 1 : 1];   // per wave: running start of each row's entries
  __shared__ uint32_t wbase[RL ? 4 : 1][RL ? kRlRows : 1];      // per wave: the rows' reserved list offsets
  const int rbase = mbase >> hshift;                  // RL: first row of the workgroup
  __shared__ float wsl[128];
  __shared__ float tsl[128];          // filter threshold of each slot's selection row
  __shared__ uint32_t pml[PM ? 128 * 16 : 1];   // page keys: [slot][page of the chunk]
  if (PM)
    for (int i = threadIdx.x; i < 128 * 16; i += 256) pml[i] = 0u;
  for (int i = threadIdx.x; i < 128; i += 256) {
    if (FILTER)
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) lcount[cc][i] = 0;
    float wv = 0.f, tv = INFINITY;
    const int ms = mbase + i;
    if (RELU && ms < M) wv = p.w[b * p.ws_[0] + (ms >> hshift) * p.ws_[1] + (ms & (p.H_I - 1)) * p.ws_[2]];
    if (FILTER && ms < M) tv = p.tau[(b * p.G_sel + (ms & (p.H_I - 1)) / HPG) * p.Nq + (ms >> hshift)];
    wsl[i] = wv;
    tsl[i] = tv;
  }
  __syncthreads();

  // RL: threshold of each of the lane's rows (row 8 mb + 2 gi + half of the
  // block: slot 32 mb + 8 gi + 4 half), the scalar entry counts of the wave,
  // and the lane's visibility offsets: key j is visible to row rbase + c +
  // half when j - (L - Nq + rbase) - half <= c, and the row exists when
  // c < Nq - rbase - half
  constexpr int NRT = RL ? NMB * (16 / HPG) : 1;
  float rthr[NRT];
  uint32_t rcnt[RL ? kRlRows : 1];
  const int rb_lim = L - p.Nq + (mbase >> hshift) + half;
  const int rb_hv = p.Nq - (mbase >> hshift) - half;
  if constexpr (RL) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int gi = 0; gi < 16 / HPG; ++gi) rthr[mb * (16 / HPG) + gi] = tsl[32 * mb + 8 * gi + 4 * half];
#pragma unroll
    for (int x = 0; x < kRlRows; ++x) rcnt[x] = 0u;
  }
  // per (slot block, head group) constants of the filter, when they fit in
  // registers: last visible key of the half-wave's slot row (-1: no row), its
  // threshold and its selection row within the request
  constexpr int G4 = 16 / HPG;
  constexpr bool HOIST = FILTER && NMB * G4 <= 8;
  constexpr int NH = HOIST ? NMB * G4 : 1;
  int hlim[NH], hlrow[NH];
  float hthr[NH];
  if constexpr (HOIST) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int gi = 0; gi < G4; ++gi) {
        const int v0 = gi * HPG;
        const int m0 = mbase + 32 * mb + 8 * (v0 >> 2) + 4 * half + (v0 & 3);
        const int r = m0 >> hshift, g = (m0 & (p.H_I - 1)) / HPG;
        const int e = mb * G4 + gi;
        hlim[e] = m0 < M ? L - p.Nq + r : -1;
        hthr[e] = tsl[(m0 - mbase) & 127];
        hlrow[e] = g * p.Nq + r;
      }
  }
  // candidate slots of chunk cc: [selection row of the request][cap]
  const int nrl = p.G_sel * p.Nq;
  auto chunk_cand = [&](int cc) -> u32x2* {
    return (u32x2*)p.cand + ((int64_t)b * p.nchunk + blockIdx.x * CPW + cc) * nrl * p.cap;
  };
  u32x2* cwc[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) cwc[cc] = FILTER ? chunk_cand(cc) : nullptr;

  // RL: the wave's staged entries to the rows' lists (wave-local: lanes
  // 0..kRlRows-1 reserve their row's space, then the entries are copied in
  // the order of the rows' running starts)
  auto rl_flush = [&]() {
    if constexpr (RL) {
      uint32_t n = 0u;
#pragma unroll
      for (int x = 0; x < kRlRows; ++x) n = lane == x ? rcnt[x] : n;
      if (lane >= kRlRows || rbase + lane >= p.Nq) n = 0u;
      const uint32_t incl = wave_prefix_incl_u32(n);
      const uint32_t ntot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (ntot > 0u) {
        const uint32_t gb = n ? atomicAdd(&p.cand_n[(int64_t)b * p.Nq + rbase + lane], n) : 0u;
        if (lane < kRlRows) {
          wpre[wid][lane] = incl - n;
          wbase[wid][lane] = gb;
        }
        if (lane == 0) wpre[wid][kRlRows] = ntot;
        __builtin_amdgcn_wave_barrier();
        for (uint32_t x = lane; x < ntot; x += 64) {
          int lo = 0;
#pragma unroll
          for (int step = kRlRows / 2; step >= 1; step >>= 1)
            if (wpre[wid][lo + step] <= x) lo += step;
          const uint32_t e = x - wpre[wid][lo];
          const uint32_t gs = wbase[wid][lo] + e;
          const int64_t rowg = (int64_t)b * p.Nq + rbase + lo;
          if (gs < (uint32_t)p.cap) {
            const u32x2 v = stage[(lo * 4 + wid) * kRlSlots + (int)e];
            p.cand[rowg * p.cap + gs] = f32_order_key(__uint_as_float(v[0]));
            p.cand_j[rowg * p.cap + gs] = v[1];
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
#pragma unroll
      for (int x = 0; x < kRlRows; ++x) rcnt[x] = 0u;
    }
  };

  u16x2 kmx[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) kmx[cc] = u16x2{0, 0};
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int cc = t / TPW, i = t % TPW;
    u32x4 cur[RW];
#pragma unroll
    for (int c = 0; c < RW; ++c) cur[c] = raw[t % PD][c];
    if (t + PD < NT) load(t + PD, raw[t % PD]);
    if (jw + cc * kMfmaChunk >= L) continue;            // the chunk lies past the context
    const int j = tile_key(t);
    // B operands (bf16) for the 4 k-steps
    u32x4 Bw[4];
    if (KT == DT_FP8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w0 = cur[s >> 1][2 * (s & 1)], w1 = cur[s >> 1][2 * (s & 1) + 1];
        Bw[s][0] = fp8x2_to_bf16x2<false>(w0);
        Bw[s][1] = fp8x2_to_bf16x2<true>(w0);
        Bw[s][2] = fp8x2_to_bf16x2<false>(w1);
        Bw[s][3] = fp8x2_to_bf16x2<true>(w1);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) Bw[s] = cur[s];
    }
    if (j < L) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t a = Bw[s][c] & 0x7FFF7FFFu;
          kmx[cc] = __builtin_elementwise_max(kmx[cc], *(const u16x2*)&a);
        }
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mb][s], *(const bf16x8*)&Bw[s], acc, 0, 0, 0);
      // epilogue: lane holds key j, slots 32*mb + 8*(v/4) + 4*half + v%4;
      // every lane of a half-wave holds the same slot row, keys differ
      float scv[G4];
#pragma unroll
      for (int gi = 0; gi < G4; ++gi) {
        float sc = 0.f;
#pragma unroll
        for (int tt = 0; tt < HPG; ++tt) {
          const int v = gi * HPG + tt;
          const float wv = RELU ? wsl[32 * mb + 8 * (v >> 2) + 4 * half + (v & 3)] : 0.f;
          // ReLU on the bit pattern: a negative float is a negative int
          const float rl = __int_as_float(max(__float_as_int(acc[v]), 0));
          sc = RELU ? fmaf(wv, rl, sc) : acc[v];
        }
        scv[gi] = sc;
      }
      if constexpr (RL) {
        // one selection group of four heads: half-wave half holds row
        // c + half of the block (c = 8 mb + 2 gi); a survivor's place in its
        // (row, wave) region is the wave's count of that row plus its rank
        // among the half-wave's survivors
        const int dj = j - rb_lim;
#pragma unroll
        for (int gi = 0; gi < G4; ++gi) {
          const int c = 8 * mb + 2 * gi;
          const bool pass = dj <= c && c < rb_hv && scv[gi] >= rthr[mb * G4 + gi];
          const uint64_t mk = ballot(pass);
          const uint32_t lo32 = (uint32_t)mk, hi32 = (uint32_t)(mk >> 32);
          const uint32_t c0 = (uint32_t)__builtin_popcount(lo32), c1 = (uint32_t)__builtin_popcount(hi32);
          const uint32_t pre = __builtin_amdgcn_mbcnt_hi(hi32, __builtin_amdgcn_mbcnt_lo(lo32, 0u));
          const uint32_t slot = half ? pre - c0 + rcnt[c + 1] : pre + rcnt[c];
          const int idx = pass ? ((c + half) * 4 + wid) * kRlSlots + (int)slot : kRlDiscard + (int)threadIdx.x;
          stage[idx] = u32x2{__float_as_uint(scv[gi]), (uint32_t)j};
          rcnt[c] += c0;
          rcnt[c + 1] += c1;
        }
      } else if constexpr (!FILTER) {
#pragma unroll
        for (int gi = 0; gi < G4; ++gi) {
          const int v0 = gi * HPG;
          const int m0 = mbase + 32 * mb + 8 * (v0 >> 2) + 4 * half + (v0 & 3);
          const int r = m0 >> hshift, g = (m0 & (p.H_I - 1)) / HPG;
          if (m0 < M && j <= L - p.Nq + r) p.scores[b * p.ss[0] + g * p.ss[1] + r * p.ss[2] + j] = scv[gi];
        }
        if constexpr (PM) {
          // page keys: maximum over the half-wave's 32 keys of each slot row,
          // merged into the tile's page
          const int pl = ((wid + 4 * i) * 32) >> p.pk_lgP;
#pragma unroll
          for (int gi = 0; gi < G4; ++gi) {
            const int v0 = gi * HPG;
            const int m0 = mbase + 32 * mb + 8 * (v0 >> 2) + 4 * half + (v0 & 3);
            uint32_t kk = (m0 < M && j <= L - p.Nq + (m0 >> hshift)) ? f32_order_key(scv[gi]) : 0u;
            kk = max(kk, (uint32_t)__builtin_amdgcn_update_dpp((int)kk, (int)kk, 0x128, 0xf, 0xf, false));
            kk = max(kk, (uint32_t)__builtin_amdgcn_update_dpp((int)kk, (int)kk, 0x124, 0xf, 0xf, false));
            kk = max(kk, (uint32_t)__builtin_amdgcn_update_dpp((int)kk, (int)kk, 0x122, 0xf, 0xf, false));
            kk = max(kk, (uint32_t)__builtin_amdgcn_update_dpp((int)kk, (int)kk, 0x121, 0xf, 0xf, false));
            const auto sw = __builtin_amdgcn_permlane16_swap(kk, kk, false, false);
            kk = max((uint32_t)sw[0], (uint32_t)sw[1]);
            if (col == 0 && kk) atomicMax(&pml[((m0 - mbase) & 127) * 16 + pl], kk);
          }
        }
      } else if constexpr (HOIST) {
        // survivors: each surviving lane takes its slot with one LDS atomic
        // (about one survivor per selection row and tile: little contention)
#pragma unroll
        for (int gi = 0; gi < G4; ++gi) {
          const int e = mb * G4 + gi;
          if (j <= hlim[e] && scv[gi] >= hthr[e]) {
            const uint32_t slot = atomicAdd(&lcount[cc][hlrow[e]], 1u);
            if (slot < (uint32_t)p.cap)
              cwc[cc][(uint32_t)hlrow[e] * (uint32_t)p.cap + slot] = u32x2{f32_order_key(scv[gi]), (uint32_t)j};
          }
        }
      } else {
        // many head groups: one half-wave append per group
        u32x2* const cw = chunk_cand(cc);
#pragma unroll
        for (int gi = 0; gi < G4; ++gi) {
          const int v0 = gi * HPG;
          const int m0 = mbase + 32 * mb + 8 * (v0 >> 2) + 4 * half + (v0 & 3);
          const int r = m0 >> hshift, g = (m0 & (p.H_I - 1)) / HPG;
          const int lim = m0 < M ? L - p.Nq + r : -1;
          const int lrow = g * p.Nq + r;
          const bool cand = j <= lim && scv[gi] >= tsl[(m0 - mbase) & 127];
          const uint64_t bm = ballot(cand);
          if (bm) {
            const uint32_t mh = (uint32_t)(bm >> (32 * half));
            uint32_t base = 0;
            if (col == 0 && mh) base = atomicAdd(&lcount[cc][lrow], (uint32_t)__popc(mh));
            base = (uint32_t)__shfl((int)base, 32 * half, 64);
            const uint32_t slot = base + (uint32_t)__popc(mh & ((1u << col) - 1u));
            if (cand && slot < (uint32_t)p.cap) {
              const uint32_t o = (uint32_t)lrow * (uint32_t)p.cap + slot;
              cw[o] = u32x2{f32_order_key(scv[gi]), (uint32_t)j};
            }
          }
        }
      }
    }
    if constexpr (RL) {
      uint32_t mx = 0u;
#pragma unroll
      for (int x = 0; x < kRlRows; ++x) mx = max(mx, rcnt[x]);
      if (mx > (uint32_t)(kRlSlots - 32)) rl_flush();
    }
  }
  if constexpr (RL) rl_flush();

  // largest |k| element of each chunk (valid keys only)
  __shared__ uint32_t red[CPW][4];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    uint32_t km = max((uint32_t)kmx[cc][0], (uint32_t)kmx[cc][1]);
    km = wave_max_u32(km);
    if (lane == 0) red[cc][wid] = km;
  }
  __syncthreads();
  if (threadIdx.x < CPW) {
    const int cx = blockIdx.x * CPW + threadIdx.x;
    const uint32_t m4 = max(max(red[threadIdx.x][0], red[threadIdx.x][1]), max(red[threadIdx.x][2], red[threadIdx.x][3]));
    if (cx < p.nchunk) p.kmax[(int64_t)b * p.nchunk + cx] = bf16_to_f32(m4);
  }
  if (PM) {
    // one key per (selection row, page of the chunk), from the row's first slot
    const int npl = kMfmaChunk >> p.pk_lgP;
    for (int e = threadIdx.x; e < 128 * npl; e += 256) {
      const int sl = e / npl, pl = e - sl * npl;
      const int m = mbase + sl;
      const int h = m & (p.H_I - 1);
      if (m >= M || h % HPG) continue;
      const int r = m >> hshift, g = h / HPG;
      const int64_t row = ((int64_t)b * p.G_sel + g) * p.Nq + r;
      const int page = (jw >> p.pk_lgP) + pl;
      if (page < p.pk_stride) p.pkeys[row * p.pk_stride + page] = pml[sl * 16 + pl];
    }
  }
  if (FILTER && !RL) {
    const int nrows = p.G_sel * p.Nq;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cx = blockIdx.x * CPW + cc;
      if (cx < p.nchunk)
        for (int i = threadIdx.x; i < nrows; i += 256)
          p.cand_n[((int64_t)b * p.nchunk + cx) * nrows + i] = lcount[cc][i];
    }
  }
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void idx_generic_kernel(IndexerParams p) {
  const int b = blockIdx.z;
  const int row = blockIdx.y;
  const int r = row / p.G_sel, g = row % p.G_sel;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  const int j0 = blockIdx.x * kGenChunk;
  const int kg = p.G_k == 1 ? 0 : g;
  const bool do_kmax = (r == 0) && (p.G_k == 1 ? g == 0 : true);
  if (j0 >= L || (!do_kmax && j0 > pos)) return;
  __shared__ float qs[4096];
  __shared__ float wsm[64];
  const int H = p.hpg, d = p.d_I;
  for (int i = threadIdx.x; i < H * d; i += blockDim.x) {
    const int h = i / d, c = i % d;
    qs[i] = load_val(p.q.p, p.q.dt, b * p.q.s[0] + r * p.q.s[1] + (g * H + h) * p.q.s[2] + c);
  }
  if ((int)threadIdx.x < H)
    wsm[threadIdx.x] = p.relu ? p.w[b * p.ws_[0] + r * p.ws_[1] + (g * H + threadIdx.x) * p.ws_[2]] : 1.f;
  __syncthreads();
  const int j = j0 + threadIdx.x;
  float kmx = 0.f;
  if (j < L) {
    const int64_t kb = b * p.k.s[0] + (int64_t)j * p.k.s[1] + kg * p.k.s[2];
    if (j <= pos) {
      float s = 0.f;
      for (int h = 0; h < H; ++h) {
        float dd = 0.f;
        for (int c = 0; c < d; ++c) dd = fmaf(qs[h * d + c], load_val(p.k.p, p.k.dt, kb + c), dd);
        s = p.relu ? fmaf(wsm[h], fmaxf(dd, 0.f), s) : dd;
      }
      p.scores[b * p.ss[0] + g * p.ss[1] + r * p.ss[2] + j] = s;
    }
    if (do_kmax)
      for (int c = 0; c < d; ++c) kmx = fmaxf(kmx, fabsf(load_val(p.k.p, p.k.dt, kb + c)));
  }
  if (do_kmax) {
    __shared__ float red[4];
    kmx = wave_max(kmx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = kmx;
    __syncthreads();
    if (threadIdx.x == 0)
      p.kmax[((int64_t)b * p.G_k + kg) * p.nchunk + blockIdx.x] =
          fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

// ----------------------------------------------------------------------------
// Row bound: |s~ - key| <= C * sum_h |w_h| * ||q_h||_1 * max|k|, where C covers
// float32 accumulation of d products in any order (u = 2^-23, conservative for
// MFMA and FMA chains alike), the ReLU/weight/head-sum chain, and the final
// rounding of the exact score to float32; plus a 25% margin.
__global__ __launch_bounds__(256) void idx_err_kernel(IndexerParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (row >= p.Nq * p.G_sel) return;
  const int r = row / p.G_sel, g = row % p.G_sel;
  const int kg = p.G_k == 1 ? 0 : g;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int nch = min(p.nchunk, (L + p.chunk - 1) / p.chunk);
  float km = 0.f;
  for (int c = lane; c < nch; c += 64) km = fmaxf(km, p.kmax[((int64_t)b * p.G_k + kg) * p.nchunk + c]);
  km = wave_max(km);
  double coef = 0.0;
  for (int e = lane; e < p.hpg * p.d_I; e += 64) {
    const int h = e / p.d_I, c = e % p.d_I;
    const double qv = fabs((double)load_val(p.q.p, p.q.dt, b * p.q.s[0] + r * p.q.s[1] + (g * p.hpg + h) * p.q.s[2] + c));
    const double wv = p.relu ? (double)p.w[b * p.ws_[0] + r * p.ws_[1] + (g * p.hpg + h) * p.ws_[2]] : 1.0;
    coef += fabs(wv) * qv;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) coef += __shfl_xor(coef, o, 64);
  if (lane) return;
  const double u = 1.0 / 8388608.0;   // 2^-23
  auto gam = [&](double n) { return n * u / (1.0 - n * u); };
  const double C = 1.25 * (gam(p.d_I + 2) + gam(p.hpg + 2) * (1.0 + gam(p.d_I + 2)) + u);
  const double e = C * coef * (double)km * (1.0 + 1e-6) + 1e-30;
  p.err[((int64_t)b * p.G_sel + g) * p.Nq + r] = (float)e * (1.0f + 1e-6f);
}

size_t indexer_ws_bytes(int B, int G_k, int ctx) {
  const int nchunk = (ctx + kGenChunk - 1) / kGenChunk;   // the larger count of the two kernels
  return (size_t)B * G_k * nchunk * sizeof(float);
}

template <int KT, int NMB, int HPG, bool RELU, int MODE>
static void launch_mfma(const IndexerParams& p, hipStream_t st) {
  // the filter (decode: few rows, long contexts) streams two chunks per
  // workgroup, three tiles in flight per wave; the other modes load a
  // chunk's tiles at once
  constexpr bool STREAM = MODE == 1 && NMB == 1;
  constexpr int CPW = STREAM ? 2 : 1;
  constexpr int PD = STREAM ? 3 : kMfmaChunk / 32 / 4;
  const int nchunk = (p.ctx + kMfmaChunk - 1) / kMfmaChunk;
  dim3 grid((nchunk + CPW - 1) / CPW, p.B, (p.Nq * p.H_I + 127) / 128);
  if constexpr (MODE == 1 && NMB == 4 && HPG == 4 && RELU) {
    if (p.cand_j) {      // per-row lists (many rows): one chunk per workgroup, its loads at once
      constexpr int kRlCpw = 1;
      hipLaunchKernelGGL((idx_mfma64_kernel<KT, NMB, HPG, RELU, MODE, kRlCpw, kMfmaChunk / 32 / 4, true>),
                         dim3((nchunk + kRlCpw - 1) / kRlCpw, p.B, (p.Nq * p.H_I + 127) / 128), dim3(256), 0, st, p);
      return;
    }
  }
  hipLaunchKernelGGL((idx_mfma64_kernel<KT, NMB, HPG, RELU, MODE, CPW, PD>), grid, dim3(256), 0, st, p);
}

template <int KT, int NMB, int MODE>
static void dispatch_hpg(const IndexerParams& p, hipStream_t st) {
  if (!p.relu) return launch_mfma<KT, NMB, 1, false, MODE>(p, st);
  if (p.hpg == 1) return launch_mfma<KT, NMB, 1, true, MODE>(p, st);
  if (p.hpg == 2) return launch_mfma<KT, NMB, 2, true, MODE>(p, st);
  return launch_mfma<KT, NMB, 4, true, MODE>(p, st);
}

template <int KT, int MODE>
static void dispatch_nmb(const IndexerParams& p, hipStream_t st) {
  const int M = p.Nq * p.H_I;
  if (M <= 32) return dispatch_hpg<KT, 1, MODE>(p, st);
  if (M <= 64) return dispatch_hpg<KT, 2, MODE>(p, st);
  return dispatch_hpg<KT, 4, MODE>(p, st);
}

// MFMA path: d_I = 64, bf16 queries, bf16/fp8 keys shared by every group,
// <= 4 heads per group, power-of-two H_I <= 128 (a slot block never splits a row)
static bool mfma_ok(const IndexerParams& p) {
  const bool pow2 = p.H_I > 0 && (p.H_I & (p.H_I - 1)) == 0;
  return p.d_I == 64 && p.q.dt == DT_BF16 && (p.k.dt == DT_BF16 || p.k.dt == DT_FP8) &&
         p.G_k == 1 && (p.hpg == 1 || p.hpg == 2 || p.hpg == 4) && pow2 && p.H_I <= 128 &&
         (int64_t)p.Nq * p.H_I <= (int64_t)128 * 65535;
}

bool index_pagekeys_ok(const IndexerParams& p, int lgP) { return mfma_ok(p) && lgP >= 5 && lgP <= 9; }

int index_chunk(const IndexerParams& p) { return mfma_ok(p) ? kMfmaChunk : kGenChunk; }

hipError_t launch_index_scores(const IndexerParams& p0, hipStream_t st) {
  IndexerParams p = p0;
  if (mfma_ok(p)) {
    p.chunk = kMfmaChunk;
    p.nchunk = (p.ctx + kMfmaChunk - 1) / kMfmaChunk;
    const bool pm = p.pkeys != nullptr;
    if (p.k.dt == DT_FP8) {
      if (pm) dispatch_nmb<DT_FP8, 2>(p, st);
      else dispatch_nmb<DT_FP8, 0>(p, st);
    } else {
      if (pm) dispatch_nmb<DT_BF16, 2>(p, st);
      else dispatch_nmb<DT_BF16, 0>(p, st);
    }
  } else {
    p.chunk = kGenChunk;
    p.nchunk = (p.ctx + kGenChunk - 1) / kGenChunk;
    dim3 grid(p.nchunk, p.Nq * p.G_sel, p.B);
    hipLaunchKernelGGL(idx_generic_kernel, grid, dim3(kGenChunk), 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.err) return e;
  dim3 g2((p.Nq * p.G_sel + 3) / 4, p.B);
  hipLaunchKernelGGL(idx_err_kernel, g2, dim3(256), 0, st, p);
  return hipGetLastError();
}

bool index_filter_ok(const IndexerParams& p) { return mfma_ok(p) && p.Nq * p.H_I <= 128; }

// per-row survivor lists: one selection group of four weighted-ReLU heads
bool index_filter_rows_ok(const IndexerParams& p) {
  return mfma_ok(p) && p.G_sel == 1 && p.H_I == 4 && p.hpg == 4 && p.relu && p.Nq * p.H_I > 128;
}

hipError_t launch_index_filter(const IndexerParams& p0, hipStream_t st) {
  IndexerParams p = p0;
  p.chunk = kMfmaChunk;
  p.nchunk = (p.ctx + kMfmaChunk - 1) / kMfmaChunk;
  if (p.k.dt == DT_FP8) dispatch_nmb<DT_FP8, 1>(p, st);
  else dispatch_nmb<DT_BF16, 1>(p, st);
  return hipGetLastError();
}

}  // namespace sp
