// Sparse attention over a visible key set S(i).
//
//  * attn_index_mfma: bf16, d = 128, index lists. One workgroup serves one
//    (request, query row, gather group, split): the Hg <= 16 query heads that
//    share both the index list and the KV head are the 16 MFMA rows, so one
//    gather of each selected K/V row serves the whole group (GQA/MQA). Each
//    wave walks tiles of 32 selected keys: K rows are loaded straight into
//    MFMA operand registers (S^T = K Q^T, 16x16x32 bf16), the softmax is
//    online in float32 (exp2 domain), V rows are staged in LDS and read back
//    transposed as the B operand of O += P V. P enters the MFMA as a bf16
//    hi/lo pair so the product keeps ~16 bits of P; with Hg <= 8 the lo part
//    rides in the unused MFMA rows. Splits of the index list are merged by
//    attn_combine with their (max, sum) pairs.
//  * attn_generic: any mode, f32 or bf16, d <= 128; one wave per (row, head):
//    lanes score 64 candidates at a time, then sweep them over the dims.
//  * Page lists (mode 4) are read as one token slot per (listed page, offset).
//    Paged K/V storage (pools of pages and a page table) is translated where
//    a key's row address is formed: logical token j of request b is row
//    j mod P of pool page table[b][j / P].
#include "common.h"
#include "internal.h"

namespace sp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- candidates
// Enumerates the visible set of one query row: t -> key position or -1.
struct Visible {
  int mode, p, count;
  const int32_t* list;   // index list (mode 1), block list (mode 3) or page list (mode 4)
  int K;                 // list length
  int g_end, w_start, bs, nb_keys, lgbs;
  int n_wg, stride, m0;    // window/global: keys before the strided ones, stride, first multiple

  SP_DEV void init(const AttnParams& a, int b, int h, int r, int pos) {
    mode = a.mode;
    p = pos;
    list = nullptr;
    K = a.K;
    if (mode == 0) {
      count = p + 1;
    } else if (mode == 5) {
      count = (p + 1) / a.bs;               // compressed entries of the complete blocks
    } else if (mode == 1) {
      const int gsel = h / (a.Hq / a.G_sel);
      list = a.sel + b * a.sels[0] + gsel * a.sels[1] + r * a.sels[2];
      count = K;
    } else if (mode == 4) {
      const int gsel = h / (a.Hq / a.G_sel);
      list = a.sel + b * a.sels[0] + gsel * a.sels[1] + r * a.sels[2];
      lgbs = a.lgbs;
      count = K;
    } else if (mode == 2) {
      g_end = min(a.n_global, p + 1);
      w_start = max(max(0, p - a.window + 1), g_end);
      count = g_end + max(0, p - w_start + 1);
      // dilated stride: the multiples of stride in [g_end, w_start)
      n_wg = count;
      stride = a.stride;
      m0 = 0;
      if (stride > 0 && w_start > 0) {
        m0 = (g_end + stride - 1) / stride;
        count += max(0, (w_start - 1) / stride - m0 + 1);
      }
    } else {
      list = a.sel + b * a.sels[0] + (h / (a.Hq / a.G_sel)) * a.sels[1] + r * a.sels[2];
      bs = a.bs;
      w_start = max(0, p - a.window + 1);
      nb_keys = K * bs;
      count = nb_keys + max(0, p - w_start + 1);
    }
    if (p < 0) count = 0;
  }
  SP_DEV int key(int t) const {
    if (mode == 0 || mode == 5) return t;
    if (mode == 1) {
      const int j = list[t];
      return (j >= 0 && j <= p) ? j : -1;
    }
    if (mode == 4) {
      const int pg = list[t >> lgbs];
      if (pg < 0) return -1;
      const int j = (pg << lgbs) + (t & ((1 << lgbs) - 1));
      return j <= p ? j : -1;
    }
    if (mode == 2) return t < g_end ? t : t < n_wg ? w_start + (t - g_end) : (m0 + (t - n_wg)) * stride;
    if (t < nb_keys) {
      const int blk = list[t / bs];
      if (blk < 0) return -1;
      const int j = blk * bs + t % bs;
      return (j < w_start && j <= p) ? j : -1;
    }
    return w_start + (t - nb_keys);
  }
};

SP_DEV float ldv(const void* p, int dt, int64_t i) {
  return dt == DT_F32 ? ((const float*)p)[i] : bf16_to_f32(((const uint16_t*)p)[i]);
}

// Element offset of key j's row of KV head kvh of request b in tensor t.
SP_DEV int64_t kv_row(const AttnParams& a, const View4& t, int b, int kvh, int j) {
  if (a.ptab) {
    const int64_t pg = a.ptab[b * a.pts + (j >> a.lgP)];
    return pg * t.s[0] + kvh * t.s[1] + (int64_t)(j & ((1 << a.lgP) - 1)) * t.s[2];
  }
  return b * t.s[0] + kvh * t.s[1] + (int64_t)j * t.s[2];
}

// ---------------------------------------------------------------- generic
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnParams a) {
  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int pos = L - a.Nq + r;
  const int kvh = h / (a.Hq / a.Hkv);
  Visible vis;
  vis.init(a, b, h, r, pos);
  __shared__ float qs[128];
  __shared__ float ps[64];
  __shared__ int js[64];
  const int64_t qb = b * a.q.s[0] + h * a.q.s[1] + r * a.q.s[2];
  for (int c = lane; c < a.d; c += 64) qs[c] = ldv(a.q.p, a.q.dt, qb + c);
  __syncthreads();
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int t0 = 0; t0 < vis.count; t0 += 64) {
    const int t = t0 + lane;
    const int j = t < vis.count ? vis.key(t) : -1;
    float z = -INFINITY;
    if (j >= 0) {
      float s = 0.f;
      const int64_t kr = kv_row(a, a.k, b, kvh, j);
      for (int c = 0; c < a.d; ++c) s = fmaf(qs[c], ldv(a.k.p, a.k.dt, kr + c), s);
      z = s * a.scale;
    }
    const float tm = wave_max(z);
    const float mn = fmaxf(m, tm);
    float pj = 0.f, alpha = 1.f;
    if (mn > -INFINITY) {
      pj = j >= 0 ? expf(z - mn) : 0.f;
      alpha = expf(m - mn);
    }
    l = l * alpha + wave_sum(pj);
    m = mn;
    acc0 *= alpha;
    acc1 *= alpha;
    ps[lane] = pj;
    js[lane] = j;
    __syncthreads();
    const int nt = min(64, vis.count - t0);
    for (int u = 0; u < nt; ++u) {
      const int ju = js[u];
      if (ju < 0) continue;
      const float pu = ps[u];
      const int64_t vr = kv_row(a, a.v, b, kvh, ju);
      if (lane < a.d) acc0 = fmaf(pu, ldv(a.v.p, a.v.dt, vr + lane), acc0);
      if (lane + 64 < a.d) acc1 = fmaf(pu, ldv(a.v.p, a.v.dt, vr + lane + 64), acc1);
    }
    __syncthreads();
  }
  float* o = a.o + b * a.os[0] + h * a.os[1] + r * a.os[2];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (lane < a.d) o[lane] = acc0 * inv;
  if (lane + 64 < a.d) o[lane + 64] = acc1 * inv;
  if (a.lse && lane == 0) a.lse[((int64_t)b * a.Hq + h) * a.Nq + r] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------- backward
// Gradients of sum(dO * O) over the same visible set, float32 (any mode):
// one wave per (row, head) walks the row's visible keys 64 at a time; lanes
// score them (s = q.k, dp = dO.v), form p = exp(s * scale - lse) and
// ds = p (dp - D) with D = dO.O; then, key by key, the lanes (one per
// dimension) add ds * scale * k to dq and add the key's dk and dv shares
// (ds * scale * q and p * dO) with float atomics, since a key's gradient
// gathers contributions from every row and head that sees it.
__global__ __launch_bounds__(256) void attn_bwd_zero_kernel(AttnParams a, AttnBwd g) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  for (int c = threadIdx.x; c < a.d; c += blockDim.x) {
    g.dk[b * g.dks[0] + h * g.dks[1] + (int64_t)j * g.dks[2] + c] = 0.f;
    g.dv[b * g.dvs[0] + h * g.dvs[1] + (int64_t)j * g.dvs[2] + c] = 0.f;
  }
}

__global__ __launch_bounds__(64) void attn_bwd_generic_kernel(AttnParams a, AttnBwd g) {
  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int pos = L - a.Nq + r;
  const int kvh = h / (a.Hq / a.Hkv);
  Visible vis;
  vis.init(a, b, h, r, pos);
  __shared__ float qs[128], dos[128], ps[64], dss[64];
  __shared__ int js[64];
  const int64_t qb = b * a.q.s[0] + h * a.q.s[1] + r * a.q.s[2];
  const float* dOr = g.dO + b * g.dos[0] + h * g.dos[1] + r * g.dos[2];
  const float* Or = g.o + b * g.os[0] + h * g.os[1] + r * g.os[2];
  float dd = 0.f;
  for (int c = lane; c < a.d; c += 64) {
    qs[c] = ldv(a.q.p, a.q.dt, qb + c);
    dos[c] = dOr[c];
    dd = fmaf(dOr[c], Or[c], dd);
  }
  const float D = wave_sum(dd);
  const float lse = g.lse[((int64_t)b * a.Hq + h) * a.Nq + r];
  __syncthreads();
  float acc0 = 0.f, acc1 = 0.f;
  const int64_t dkb = b * g.dks[0] + kvh * g.dks[1];
  const int64_t dvb = b * g.dvs[0] + kvh * g.dvs[1];
  if (lse > -INFINITY) {
    for (int t0 = 0; t0 < vis.count; t0 += 64) {
      const int t = t0 + lane;
      const int j = t < vis.count ? vis.key(t) : -1;
      float p = 0.f, ds = 0.f;
      if (j >= 0) {
        const int64_t kr = kv_row(a, a.k, b, kvh, j), vr = kv_row(a, a.v, b, kvh, j);
        float sdot = 0.f, dp = 0.f;
        for (int c = 0; c < a.d; ++c) {
          sdot = fmaf(qs[c], ldv(a.k.p, a.k.dt, kr + c), sdot);
          dp = fmaf(dos[c], ldv(a.v.p, a.v.dt, vr + c), dp);
        }
        p = expf(sdot * a.scale - lse);
        ds = p * (dp - D) * a.scale;
      }
      ps[lane] = p;
      dss[lane] = ds;
      js[lane] = j;
      __syncthreads();
      const int nt = min(64, vis.count - t0);
      for (int u = 0; u < nt; ++u) {
        const int ju = js[u];
        if (ju < 0) continue;
        const float pu = ps[u], dsu = dss[u];
        const int64_t kr = kv_row(a, a.k, b, kvh, ju);
        if (lane < a.d) {
          acc0 = fmaf(dsu, ldv(a.k.p, a.k.dt, kr + lane), acc0);
          atomicAdd(&g.dk[dkb + (int64_t)ju * g.dks[2] + lane], dsu * qs[lane]);
          atomicAdd(&g.dv[dvb + (int64_t)ju * g.dvs[2] + lane], pu * dos[lane]);
        }
        if (lane + 64 < a.d) {
          acc1 = fmaf(dsu, ldv(a.k.p, a.k.dt, kr + lane + 64), acc1);
          atomicAdd(&g.dk[dkb + (int64_t)ju * g.dks[2] + lane + 64], dsu * qs[lane + 64]);
          atomicAdd(&g.dv[dvb + (int64_t)ju * g.dvs[2] + lane + 64], pu * dos[lane + 64]);
        }
      }
      __syncthreads();
    }
  }
  float* dq = g.dq + b * g.dqs[0] + h * g.dqs[1] + r * g.dqs[2];
  if (lane < a.d) dq[lane] = acc0;
  if (lane + 64 < a.d) dq[lane + 64] = acc1;
}

size_t attn_bwd_ws_bytes(const AttnParams& a) {
  const int ns = attn_bwd_tile_ok(a) ? attn_bwd_slots(a) : 0;
  if (ns == 0) return 0;
  return (size_t)a.B * a.Hq * ((a.ctx + 63) / 64) * ns * (64 * 128 * 2) * sizeof(float);
}

hipError_t launch_attention_bwd(const AttnParams& a, const AttnBwd& g, hipStream_t st) {
  const int zr = attn_bwd_zero_rows(a, g);
  if (zr > 0) {
    hipLaunchKernelGGL(attn_bwd_zero_kernel, dim3(zr, a.Hkv, a.B), dim3(128), 0, st, a, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (attn_bwd_tile_ok(a)) return launch_attn_bwd_tile(a, g, st);
  hipLaunchKernelGGL(attn_bwd_generic_kernel, dim3(a.Nq, a.Hq, a.B), dim3(64), 0, st, a, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- MFMA gather
constexpr int kVStride = 132;   // per-wave staging area: 32 rows of 264 B (rows are used at 256 B)
typedef short v4i16 __attribute__((ext_vector_type(4)));

struct SplitInfo {
  int nsplit, per;   // splits per row, list entries per split (multiple of 32)
};
constexpr int kMaxTilesPerWave = 16;   // 32-entry tiles per wave of one split

template <bool PACKLO, bool PIPE, bool PAGED>
__global__ __launch_bounds__(256) void attn_index_mfma_kernel(AttnParams a, int Hg, SplitInfo si,
                                                              float* part) {
  const int split = blockIdx.x;
  const int ngg = a.Hq / Hg;
  const int rowid = blockIdx.y;             // (b, r, gg) flattened
  const int gg = rowid % ngg;
  const int r = (rowid / ngg) % a.Nq;
  const int b = rowid / (ngg * a.Nq);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int qq = lane >> 4, c16 = lane & 15;
  const int h0 = gg * Hg;
  const int kvh = h0 / (a.Hq / a.Hkv);
  const int gsel = h0 / (a.Hq / a.G_sel);
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int pos = L - a.Nq + r;
  const int32_t* list = a.sel + b * a.sels[0] + gsel * a.sels[1] + r * a.sels[2];
  const int t_begin = split * si.per;
  const int t_end = min(a.K, t_begin + si.per);

  __shared__ __attribute__((aligned(16))) uint16_t vs[4][32 * kVStride];
  __shared__ int idxs[4][kMaxTilesPerWave * 32];

  // Q^T as the B operand: lane holds head c16, dims 8 * (4 ks + qq) + v for
  // k-step ks (the K rows below use the same order of the dims, so the four
  // lanes of a key row read 64 contiguous bytes per load instruction)
  bf16x8 Qb[4];
  {
    const int hh = c16;
    if (hh < Hg) {
      const uint16_t* qp = (const uint16_t*)a.q.p + b * a.q.s[0] + (h0 + hh) * a.q.s[1] + r * a.q.s[2] + 8 * qq;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Qb[ks] = *(const bf16x8*)(qp + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Qb[ks] = (bf16x8){};
    }
  }
  const float c = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // key rows: list entries become logical tokens j (page lists: one entry per
  // token slot), then, with paged storage, pool tokens (pool page << lgP | row)
  const uint16_t* kbase = (const uint16_t*)a.k.p + (PAGED ? 0 : b * a.k.s[0]) + kvh * a.k.s[1];
  const uint16_t* vbase = (const uint16_t*)a.v.p + (PAGED ? 0 : b * a.v.s[0]) + kvh * a.v.s[1];
  const int pmask = (1 << a.lgP) - 1;
  auto krow = [&](int j) -> int64_t {
    return PAGED ? (int64_t)(j >> a.lgP) * a.k.s[0] + (int64_t)(j & pmask) * a.k.s[2] : (int64_t)j * a.k.s[2];
  };
  auto vrow = [&](int j) -> int64_t {
    return PAGED ? (int64_t)(j >> a.lgP) * a.v.s[0] + (int64_t)(j & pmask) * a.v.s[2] : (int64_t)j * a.v.s[2];
  };

  // this wave's tiles of 32 list entries: t_begin + 32 wid + 128 i; all their
  // entries are loaded at once
  const int first = t_begin + 32 * wid;
  const int ntw = first < t_end ? (t_end - first + 127) / 128 : 0;
  int* wix = idxs[wid];
  for (int e = lane; e < ntw * 32; e += 64) {
    const int t = first + 128 * (e >> 5) + (e & 31);
    int j = -1;
    if (t < t_end) {
      if (a.mode == 4) {
        const int pg = list[t >> a.lgbs];
        j = pg < 0 ? -1 : (pg << a.lgbs) + (t & ((1 << a.lgbs) - 1));
      } else {
        j = list[t];
      }
    }
    if (j > pos) j = -1;
    if (PAGED && j >= 0) j = (a.ptab[b * a.pts + (j >> a.lgP)] << a.lgP) | (j & pmask);
    wix[e] = j;
  }
  __builtin_amdgcn_wave_barrier();

  // K rows for the two 16-key subtiles (row c16 and 16 + c16; k-step ks:
  // dims 8 * (4 ks + qq) .. +8, so one instruction reads 64 contiguous bytes
  // of each row) and V rows (chunk u: key qq + 4u, 16-byte column c16) of tile i
  auto issue = [&](int i, u32x4 (&kr)[2][4], u32x4 (&vr)[8]) {
    const int* ix = wix + 32 * i;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      int j = ix[16 * st + c16];
      j = j < 0 ? 0 : j;
      const uint16_t* kp = kbase + krow(j) + 8 * qq;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[st][ks] = *(const u32x4*)(kp + 32 * ks);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int j = ix[qq + 4 * u];
      j = j < 0 ? 0 : j;
      vr[u] = *(const u32x4*)(vbase + vrow(j) + 8 * c16);
    }
  };

  auto compute = [&](int i, const u32x4 (&kr)[2][4], const u32x4 (&vr)[8]) {
    const int* ix = wix + 32 * i;
    // S^T = K Q^T
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&kr[0][ks], Qb[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&kr[1][ks], Qb[ks], S1, 0, 0, 0);
    }
    // lane: head c16, keys 4*qq + v (S0) and 16 + 4*qq + v (S1)
    float z[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      z[v] = ix[4 * qq + v] >= 0 ? S0[v] * c : -INFINITY;
      z[4 + v] = ix[16 + 4 * qq + v] >= 0 ? S1[v] * c : -INFINITY;
    }
    float tm = z[0];
#pragma unroll
    for (int v = 1; v < 8; ++v) tm = fmaxf(tm, z[v]);
    tm = rows4_max(tm);
    const float mn = fmaxf(m, tm);
    // lazy rescale: P is formed against the reference maximum m, which moves
    // (rescaling O and l) only when some head's maximum has grown past it by
    // more than 8 (log2 units), so P stays below 2^8 (exact in the bf16
    // hi/lo pair as before, far from float32 overflow); the branch is the
    // same for the whole wave, and after the first tiles it is rarely taken
    const bool up = __any(mn > m + 8.f);
    const float mr = up ? mn : m;
    float alpha = 1.f, ps = 0.f;
    float pv[8];
    if (mr > -INFINITY) {
      if (up) alpha = exp2f(m - mr);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        pv[v] = exp2f(z[v] - mr);
        ps += pv[v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) pv[v] = 0.f;
    }
    ps = rows4_sum(ps);
    l = l * alpha + ps;
    m = mr;
    // rescale O: lane holds rows (heads) 4*qq + v; alpha of head hh lives in
    // lane hh (read with readlane, then picked by the lane's row group; with
    // PACKLO rows 8..15 repeat heads 0..7)
#pragma unroll
    for (int v = 0; v < 4 && up; ++v) {
      const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), v));
      const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 4 + v));
      float av;
      if (PACKLO) {
        av = (qq & 1) ? a1 : a0;
      } else {
        const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 8 + v));
        const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 12 + v));
        av = qq == 0 ? a0 : qq == 1 ? a1 : qq == 2 ? a2 : a3;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) O[nt][v] *= av;
    }
    // P as the A operand (row = head c16, k = 8*qq + v <-> key mapping above)
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int v2 = 0; v2 < 4; ++v2) {
      const float x0 = pv[2 * v2], x1 = pv[2 * v2 + 1];
      const uint32_t h0b = f32_to_bf16_rne(x0), h1b = f32_to_bf16_rne(x1);
      const float r0 = x0 - bf16_to_f32(h0b), r1 = x1 - bf16_to_f32(h1b);
      ph[v2] = h0b | (h1b << 16);
      pl[v2] = f32_to_bf16_rne(r0) | (f32_to_bf16_rne(r1) << 16);
    }
    // pv[0..3] are keys 4qq+0..3 (k = 8qq+0..3), pv[4..7] keys 16+4qq+0..3 (k = 8qq+4..7)
    u32x4 Ahi, Alo;
    if (PACKLO) {
      // rows 0..7: hi of heads 0..7; rows 8..15: lo of heads 0..7 (from lane - 8
      // of the same 16-lane row: DPP row_shr:8)
      uint32_t plo_src[4];
#pragma unroll
      for (int v2 = 0; v2 < 4; ++v2)
        plo_src[v2] = (uint32_t)__builtin_amdgcn_update_dpp((int)pl[v2], (int)pl[v2], 0x118, 0xf, 0xf, false);
#pragma unroll
      for (int v2 = 0; v2 < 4; ++v2) Ahi[v2] = c16 < 8 ? ph[v2] : plo_src[v2];
    } else {
#pragma unroll
      for (int v2 = 0; v2 < 4; ++v2) {
        Ahi[v2] = ph[v2];
        Alo[v2] = pl[v2];
      }
    }
    // stage V rows in LDS row-major (256 B per key row), 16-byte chunk c of
    // row r at chunk c ^ (r mod 16), so that the rows read together by the
    // transposed reads below spread over the banks
    uint16_t* vw = &vs[wid][0];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = qq + 4 * u;
      *(u32x4*)&vw[row * 128 + 8 * (c16 ^ (row & 15))] = vr[u];
    }
    __builtin_amdgcn_wave_barrier();
    // B operand (column dim 16 nt + c16, k = 8 qq + v <-> keys 4 qq + v and
    // 16 + 4 qq + v - 4) by two LDS transposed reads per nt: lane (qq, j) of
    // a 16-lane group points at key row 4 qq + j / 4 (+16), dims 16 nt +
    // 4 (j mod 4) .. +3, and receives dim 16 nt + j of the group's four rows
    const int trow = 4 * qq + (c16 >> 2);
    const int tsub = 4 * (c16 & 3);                 // dim offset within the 16-dim slab
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int lchunk = 2 * nt + (tsub >> 3);      // logical 16-byte chunk of the row
      const int within = tsub & 7;                  // 16-bit words into the chunk
      const uint16_t* p0 = &vw[trow * 128 + 8 * (lchunk ^ (trow & 15)) + within];
      const uint16_t* p1 = &vw[(trow + 16) * 128 + 8 * (lchunk ^ ((trow + 16) & 15)) + within];
      const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
      const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
      u32x4 Bv;
      Bv[0] = (uint32_t)(uint16_t)r0[0] | ((uint32_t)(uint16_t)r0[1] << 16);
      Bv[1] = (uint32_t)(uint16_t)r0[2] | ((uint32_t)(uint16_t)r0[3] << 16);
      Bv[2] = (uint32_t)(uint16_t)r1[0] | ((uint32_t)(uint16_t)r1[1] << 16);
      Bv[3] = (uint32_t)(uint16_t)r1[2] | ((uint32_t)(uint16_t)r1[3] << 16);
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&Ahi, *(const bf16x8*)&Bv, O[nt], 0, 0, 0);
      if (!PACKLO)
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&Alo, *(const bf16x8*)&Bv, O[nt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  if constexpr (PIPE) {
    // two register sets: the rows of tile i + 1 are in flight while tile i is
    // computed (few rows: one workgroup per CU, latency hidden in the wave)
    u32x4 kA[2][4], vA[8], kB[2][4], vB[8];
    if (ntw > 0) issue(0, kA, vA);
    for (int i = 0; i < ntw; i += 2) {
      if (i + 1 < ntw) issue(i + 1, kB, vB);
      compute(i, kA, vA);
      if (i + 1 >= ntw) break;
      if (i + 2 < ntw) issue(i + 2, kA, vA);
      compute(i + 1, kB, vB);
    }
  } else {
    // many rows: one register set, latency hidden by occupancy
    u32x4 kA[2][4], vA[8];
    for (int i = 0; i < ntw; ++i) {
      issue(i, kA, vA);
      compute(i, kA, vA);
    }
  }

  // merge the 4 waves through LDS (reuses the V staging area)
  __syncthreads();
  float* red = (float*)&vs[0][0];                 // [4][16][128] partial O
  float* ml = red + 4 * 16 * 128;                 // [4][16][2]
  static_assert(sizeof(float) * (4 * 16 * 128 + 4 * 16 * 2) <= sizeof(uint16_t) * 4 * 32 * kVStride,
                "merge area must fit in the V staging buffer");
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wid * 16 + 4 * qq + v) * 128 + 16 * nt + c16] = O[nt][v];
  if (qq == 0) {
    ml[(wid * 16 + c16) * 2 + 0] = m;
    ml[(wid * 16 + c16) * 2 + 1] = l;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Hg * 128; e += 256) {
    const int hh = e >> 7, dd = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * 16 + hh) * 2]);
    float Ls = 0.f, Os = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = ml[(w * 16 + hh) * 2];
        const float f = mw > -INFINITY ? exp2f(mw - M) : 0.f;
        Ls += ml[(w * 16 + hh) * 2 + 1] * f;
        float ov = red[(w * 16 + hh) * 128 + dd];
        if (PACKLO) ov += red[(w * 16 + hh + 8) * 128 + dd];
        Os += ov * f;
      }
    }
    if (si.nsplit == 1) {
      float* o = a.o + b * a.os[0] + (h0 + hh) * a.os[1] + r * a.os[2];
      o[dd] = Ls > 0.f ? Os / Ls : 0.f;
      if (a.lse && dd == 0)
        a.lse[((int64_t)b * a.Hq + h0 + hh) * a.Nq + r] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
    } else {
      float* pp = part + (((int64_t)rowid * si.nsplit + split) * Hg + hh) * 130;
      pp[dd] = Os;
      if (dd == 0) {
        pp[128] = M;
        pp[129] = Ls;
      }
    }
  }
}

// merge splits: one workgroup of 128 threads per (b, r, gather group, head).
// Up to kCombineRegs splits, every thread loads every split's (max, sum)
// pair and its own output element in one round (split indices past the last
// are clamped and weighted 0, so no load waits on a condition) and merges in
// registers; more splits take a loop.
constexpr int kCombineRegs = 8;
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnParams a, int Hg, SplitInfo si,
                                                           const float* part) {
  const int ngg = a.Hq / Hg;
  const int rowid = blockIdx.x, hh = blockIdx.y;
  const int gg = rowid % ngg;
  const int r = (rowid / ngg) % a.Nq;
  const int b = rowid / (ngg * a.Nq);
  const int dd = threadIdx.x;
  const float* base = part + ((int64_t)rowid * si.nsplit * Hg + hh) * 130;
  const int64_t sstride = (int64_t)Hg * 130;
  float M = -INFINITY, Ls = 0.f, Os = 0.f;
  if (si.nsplit <= kCombineRegs) {
    float mv[kCombineRegs], lv[kCombineRegs], ov[kCombineRegs];
#pragma unroll
    for (int s = 0; s < kCombineRegs; ++s) {
      const float* ps = base + min(s, si.nsplit - 1) * sstride;
      mv[s] = ps[128];
      lv[s] = ps[129];
      ov[s] = ps[dd];
    }
#pragma unroll
    for (int s = 0; s < kCombineRegs; ++s)
      if (s < si.nsplit) M = fmaxf(M, mv[s]);
    if (M > -INFINITY) {
#pragma unroll
      for (int s = 0; s < kCombineRegs; ++s) {
        const float f = (s < si.nsplit && mv[s] > -INFINITY) ? exp2f(mv[s] - M) : 0.f;
        Ls += lv[s] * f;
        Os += ov[s] * f;
      }
    }
  } else {
    for (int s = 0; s < si.nsplit; ++s) M = fmaxf(M, base[s * sstride + 128]);
    if (M > -INFINITY)
      for (int s = 0; s < si.nsplit; ++s) {
        const float mv = base[s * sstride + 128];
        const float f = mv > -INFINITY ? exp2f(mv - M) : 0.f;
        Ls += base[s * sstride + 129] * f;
        Os += base[s * sstride + dd] * f;
      }
  }
  const int h = gg * Hg + hh;
  float* o = a.o + b * a.os[0] + h * a.os[1] + r * a.os[2];
  o[dd] = (M > -INFINITY && Ls > 0.f) ? Os / Ls : 0.f;
  if (a.lse && dd == 0)
    a.lse[((int64_t)b * a.Hq + h) * a.Nq + r] = (M > -INFINITY && Ls > 0.f) ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- dispatch
static int gather_group(const AttnParams& a) {
  const int per_kv = a.Hq / a.Hkv, per_sel = a.Hq / a.G_sel;
  return per_kv < per_sel ? per_kv : per_sel;
}

static bool mfma_index_ok(const AttnParams& a) {
  return (a.mode == 1 || a.mode == 4) && a.q.dt == DT_BF16 && a.d == 128 && gather_group(a) <= 16;
}

static SplitInfo pick_split(const AttnParams& a, int Hg) {
  // Few rows (decode): enough splits for one workgroup per CU, but at least
  // two tiles per wave so that loads overlap compute. Many rows: no split
  // unless a split would exceed the tiles a wave can list.
  const int rows = a.B * a.Nq * (a.Hq / Hg);
  const int tiles = (a.K + 31) / 32;
  const int minsplit = (tiles + 4 * kMaxTilesPerWave - 1) / (4 * kMaxTilesPerWave);
  int ns = (256 + rows - 1) / rows;
  const int maxs = tiles / 8 > 1 ? tiles / 8 : 1;
  if (ns > maxs) ns = maxs;
  if (ns > 64) ns = 64;
  if (ns < minsplit) ns = minsplit;
  if (ns < 1) ns = 1;
  const int per_tiles = (tiles + ns - 1) / ns;
  SplitInfo si;
  si.per = per_tiles * 32;
  si.nsplit = (a.K + si.per - 1) / si.per;
  return si;
}

size_t attn_ws_bytes(const AttnParams& a) {
  if (attn_blocks_ok(a)) return attn_blocks_ws_bytes(a);
  if (!mfma_index_ok(a)) return 0;
  const int Hg = gather_group(a);
  const SplitInfo si = pick_split(a, Hg);
  if (si.nsplit == 1) return 0;
  const size_t rows = (size_t)a.B * a.Nq * (a.Hq / Hg);
  return rows * si.nsplit * Hg * 130 * sizeof(float);
}

hipError_t launch_attention(const AttnParams& a, hipStream_t st) {
  if (mfma_index_ok(a)) {
    const int Hg = gather_group(a);
    const SplitInfo si = pick_split(a, Hg);
    const int rows = a.B * a.Nq * (a.Hq / Hg);
    float* part = (float*)a.ws;
    dim3 grid(si.nsplit, rows);
    const bool pipe = (int64_t)rows * si.nsplit <= 1024;   // at most ~4 workgroups per CU
#define SP_ATTN_MFMA(PL, PI, PG) \
  hipLaunchKernelGGL((attn_index_mfma_kernel<PL, PI, PG>), grid, dim3(256), 0, st, a, Hg, si, part)
    const bool paged = a.ptab != nullptr;
    if (Hg <= 8) {
      if (pipe) { if (paged) SP_ATTN_MFMA(true, true, true); else SP_ATTN_MFMA(true, true, false); }
      else { if (paged) SP_ATTN_MFMA(true, false, true); else SP_ATTN_MFMA(true, false, false); }
    } else {
      if (pipe) { if (paged) SP_ATTN_MFMA(false, true, true); else SP_ATTN_MFMA(false, true, false); }
      else { if (paged) SP_ATTN_MFMA(false, false, true); else SP_ATTN_MFMA(false, false, false); }
    }
#undef SP_ATTN_MFMA
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || si.nsplit == 1) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(rows, Hg), dim3(128), 0, st, a, Hg, si,
                       (const float*)part);
    return hipGetLastError();
  }
  if (attn_blocks_ok(a)) return launch_attn_blocks(a, st);
  if (attn_tile_ok(a)) return launch_attn_tile(a, st);
  dim3 grid(a.Nq, a.Hq, a.B);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace sp
