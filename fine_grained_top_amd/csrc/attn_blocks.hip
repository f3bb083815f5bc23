// Block-centric attention for per-row selected blocks (BLOCKS mode), bf16,
// d = 128.
//
// With block choices that differ per row and head, the union of the blocks
// of a few rows covers most of the context, so a query-tiled kernel would do
// nearly dense work. Here the work is organized by key block instead: the
// rows that chose a block are gathered and attend to that block once, and
// each row's partial results are merged with its window part by their
// softmax statistics (the decomposition MoBA uses: attention over a union of
// disjoint key sets is the log-sum-exp merge of the parts).
//
// Block lists belong to selection groups (one per query head, or one per
// GQA group whose query heads share a KV head and a list, as MSA's index
// branch picks blocks per group); the bookkeeping runs per (request, group)
// and a work item serves every query head of its group, so a chosen key
// block is staged once for the group (KV-outer, queries gathered):
//
//   count   per 256-row chunk: which (row, slot) entries contribute (valid,
//           not a repeat of an earlier slot, some key before the row's window
//           and not after the row), a per-block histogram and each entry's
//           rank within its chunk's bin
//   scan    per (request, group): per-chunk offsets of every block's list,
//           list bases, work items per block and their prefix
//   table   the flat list of work items (request-group, block, row chunk)
//   scatter each contributing (row, slot) into its block's row list
//   attn    one workgroup per work item: the block's keys staged in LDS, the
//           item's 64 / hpg rows of each of the group's hpg query heads
//           gathered as the 64 MFMA rows, S^T = K Q^T and O += P V on MFMA,
//           partial (m, l, O) per (row, head, slot)
//   window  the tiled kernel in window mode (O and LSE of the window part)
//   combine per row: merge the window part with the block partials
//
// Keys in both a chosen block and the row's window belong to the window part
// only, so every visible key is counted once.
#include "common.h"
#include "internal.h"

typedef short v4i16 __attribute__((ext_vector_type(4)));

namespace sp {

constexpr int kBcRows = 256;     // rows per count/scatter workgroup
constexpr int kBcTM = 64;        // rows per attention work item
constexpr int kBcMaxBlocks = 2048;
constexpr int kBcKs = 136;       // K tile row stride in 16-bit words
constexpr float kBcLog2e = 1.4426950408889634f;
constexpr float kBcLn2 = 0.6931471805599453f;
// One (row, head, slot) partial: m, l and a scale (4 words with a pad), then
// the 128 dims of the normalized output O / l as 16-bit fixed point relative
// to the scale (the largest |O / l| of the partial): 272 bytes instead of
// 520 for float32. The merged output is a convex combination of the
// normalized partials, so its error from this rounding is at most
// scale / 65534, below 1e-4 for values of |v| up to 6.
constexpr int kBcPart = 4 + 64;   // 32-bit words
constexpr int kBcListMax = 32;    // list slots held in registers by count/scatter

struct BcWs {
  int32_t* rank;      // [B*G][Nq][nb]: rank within the chunk's bin, -1 = no contribution
  int32_t* hist;      // [B*G][nch][nbk]: chunk counts, then exclusive offsets over chunks
  int32_t* tot;       // [B*G][nbk]: rows per block
  int32_t* lbase;     // [B*G][nbk]: list base of each block
  int32_t* ioff;      // [B*G][nbk]: first work item of each block within its (request, group)
  int32_t* icnt;      // [B*G]: work items per (request, group)
  int32_t* nitems;    // [1]: total work items
  uint32_t* item_bk;  // [maxitems]: (request, group) * nbk + block
  uint32_t* item_c;   // [maxitems]: row chunk of the block's list
  uint32_t* list;     // [B*G][Nq*nb]: row | slot << 24
  float* part;        // [B*Hq][Nq][nb][kBcPart]: m, l, scale, pad, 128 x int16 O / l
  float* lse_w;       // [B*Hq][Nq]: LSE of the window part
  int nch, nbk, maxitems;
  int hpg, rpi;       // query heads per selection group, rows per work item (64 / hpg)
};

static int bc_max_items(const AttnParams& a, int nbk) {
  const int64_t bg = (int64_t)a.B * a.G_sel;
  const int rpi = kBcTM / (a.Hq / a.G_sel);
  return (int)(bg * (((int64_t)a.Nq * a.K + rpi - 1) / rpi + nbk));
}

static BcWs bc_layout(const AttnParams& a, void* base, size_t* bytes) {
  BcWs w{};
  w.nbk = (a.ctx + a.bs - 1) / a.bs;
  w.nch = (a.Nq + kBcRows - 1) / kBcRows;
  w.maxitems = bc_max_items(a, w.nbk);
  w.hpg = a.Hq / a.G_sel;
  w.rpi = kBcTM / w.hpg;
  const int64_t bh = (int64_t)a.B * a.Hq;
  const int64_t bg = (int64_t)a.B * a.G_sel;
  const int64_t ent = bh * a.Nq * a.K;
  const int64_t gent = bg * a.Nq * a.K;
  size_t off = 0;
  auto take = [&](size_t n) {
    char* p = (char*)base + off;
    off += (n + 255) & ~(size_t)255;
    return (void*)p;
  };
  w.part = (float*)take((size_t)ent * kBcPart * sizeof(float));
  w.rank = (int32_t*)take((size_t)gent * 4);
  w.list = (uint32_t*)take((size_t)gent * 4);
  w.hist = (int32_t*)take((size_t)bg * w.nch * w.nbk * 4);
  w.tot = (int32_t*)take((size_t)bg * w.nbk * 4);
  w.lbase = (int32_t*)take((size_t)bg * w.nbk * 4);
  w.ioff = (int32_t*)take((size_t)bg * w.nbk * 4);
  w.icnt = (int32_t*)take((size_t)bg * 4);
  w.nitems = (int32_t*)take(4);
  w.item_bk = (uint32_t*)take((size_t)w.maxitems * 4);
  w.item_c = (uint32_t*)take((size_t)w.maxitems * 4);
  w.lse_w = (float*)take((size_t)bh * a.Nq * 4);
  if (bytes) *bytes = off;
  return w;
}

// a selection group's query heads (a power of two up to 64 of them) share
// one KV head
bool attn_blocks_ok(const AttnParams& a) {
  const int hpg = a.Hq / a.G_sel;
  return a.mode == 3 && attn_tile_ok(a) && (a.ctx + a.bs - 1) / a.bs <= kBcMaxBlocks && a.K <= 255 &&
         a.Nq < (1 << 24) && hpg <= kBcTM && (hpg & (hpg - 1)) == 0 && (a.Hq / a.Hkv) % hpg == 0;
}

size_t attn_blocks_ws_bytes(const AttnParams& a) {
  size_t bytes = 0;
  bc_layout(a, nullptr, &bytes);
  return bytes;
}

// does slot s of a row contribute: a valid block, not a repeat of an earlier
// slot, with some key at or before the row's position and before its window
SP_DEV bool bc_contributes(const AttnParams& a, const int32_t* sel, int s, int nbk, int p, int wstart) {
  const int blk = sel[s * a.sels[3]];
  if (blk < 0 || blk >= nbk) return false;
  for (int s2 = 0; s2 < s; ++s2)
    if (sel[s2 * a.sels[3]] == blk) return false;
  const int lo = blk * a.bs;
  const int hi = min(min(lo + a.bs - 1, p), wstart - 1);
  return hi >= lo;
}

// a row's block list into registers (entries past K read as -1): four
// entries per load when the list is contiguous and 16-byte aligned
SP_DEV void bc_load_list(const AttnParams& a, const int32_t* sel, int (&blk)[kBcListMax]) {
  if (a.sels[3] == 1 && (a.K & 3) == 0 && (((uintptr_t)sel) & 15) == 0) {
#pragma unroll
    for (int s4 = 0; s4 < kBcListMax / 4; ++s4) {
      int4 v = make_int4(-1, -1, -1, -1);
      if (4 * s4 < a.K) v = *(const int4*)(sel + 4 * s4);
      blk[4 * s4] = v.x;
      blk[4 * s4 + 1] = v.y;
      blk[4 * s4 + 2] = v.z;
      blk[4 * s4 + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int s = 0; s < kBcListMax; ++s) blk[s] = s < a.K ? sel[s * a.sels[3]] : -1;
  }
}

__global__ __launch_bounds__(kBcRows) void bc_count_kernel(AttnParams a, BcWs w) {
  __shared__ int hist[kBcMaxBlocks];
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.G_sel + g;
  for (int i = threadIdx.x; i < w.nbk; i += kBcRows) hist[i] = 0;
  __syncthreads();
  const int r = ch * kBcRows + threadIdx.x;
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  if (r < a.Nq) {
    const int p = L - a.Nq + r;
    const int wstart = p - a.window + 1;
    const int32_t* sel = a.sel + b * a.sels[0] + g * a.sels[1] + (int64_t)r * a.sels[2];
    int32_t* rk = w.rank + ((int64_t)bh * a.Nq + r) * a.K;
    if (a.K <= kBcListMax) {
      // the list in registers; the same contribution rule as bc_contributes
      int blk[kBcListMax], rv[kBcListMax];
      bc_load_list(a, sel, blk);
#pragma unroll
      for (int s = 0; s < kBcListMax; ++s) {
        bool c = s < a.K && p >= 0 && blk[s] >= 0 && blk[s] < w.nbk;
#pragma unroll
        for (int s2 = 0; s2 < s; ++s2) c = c && blk[s2] != blk[s];
        const int lo = blk[s] * a.bs;
        c = c && min(min(lo + a.bs - 1, p), wstart - 1) >= lo;
        rv[s] = c ? atomicAdd(&hist[blk[s]], 1) : -1;
      }
      if ((a.K & 3) == 0) {
#pragma unroll
        for (int s4 = 0; s4 < kBcListMax / 4; ++s4)
          if (4 * s4 < a.K) *(int4*)(rk + 4 * s4) = make_int4(rv[4 * s4], rv[4 * s4 + 1], rv[4 * s4 + 2], rv[4 * s4 + 3]);
      } else {
#pragma unroll
        for (int s = 0; s < kBcListMax; ++s)
          if (s < a.K) rk[s] = rv[s];
      }
    } else {
      for (int s = 0; s < a.K; ++s) {
        int v = -1;
        if (p >= 0 && bc_contributes(a, sel, s, w.nbk, p, wstart)) v = atomicAdd(&hist[sel[s * a.sels[3]]], 1);
        rk[s] = v;
      }
    }
  }
  __syncthreads();
  int32_t* hg = w.hist + ((int64_t)bh * w.nch + ch) * w.nbk;
  for (int i = threadIdx.x; i < w.nbk; i += kBcRows) hg[i] = hist[i];
}

// per (request, head): chunk offsets per block, totals, list bases, work items
__global__ __launch_bounds__(256) void bc_scan_kernel(AttnParams a, BcWs w) {
  constexpr int T = 256;
  __shared__ int sc[T];
  __shared__ int sci[T];
  const int bh = blockIdx.x;
  const int per = (w.nbk + T - 1) / T;           // <= 8 blocks per thread
  int tot[8], items[8];
  int st = 0, si = 0;
  for (int u = 0; u < per; ++u) {
    const int blk = threadIdx.x * per + u;
    int run = 0;
    if (blk < w.nbk) {
      for (int c = 0; c < w.nch; ++c) {
        int32_t* hp = w.hist + ((int64_t)bh * w.nch + c) * w.nbk + blk;
        const int v = *hp;
        *hp = run;
        run += v;
      }
    }
    tot[u] = run;
    items[u] = (run + w.rpi - 1) / w.rpi;
    st += run;
    si += items[u];
  }
  sc[threadIdx.x] = st;
  sci[threadIdx.x] = si;
  __syncthreads();
  // exclusive prefix over threads (256 entries; one thread does it)
  if (threadIdx.x == 0) {
    int r0 = 0, r1 = 0;
    for (int t = 0; t < T; ++t) {
      const int v0 = sc[t], v1 = sci[t];
      sc[t] = r0;
      sci[t] = r1;
      r0 += v0;
      r1 += v1;
    }
    w.icnt[bh] = r1;
  }
  __syncthreads();
  int lb = sc[threadIdx.x], io = sci[threadIdx.x];
  for (int u = 0; u < per; ++u) {
    const int blk = threadIdx.x * per + u;
    if (blk < w.nbk) {
      w.tot[(int64_t)bh * w.nbk + blk] = tot[u];
      w.lbase[(int64_t)bh * w.nbk + blk] = lb;
      w.ioff[(int64_t)bh * w.nbk + blk] = io;
    }
    lb += tot[u];
    io += items[u];
  }
}

// the flat work-item table; every (request, head) adds the items before it
__global__ __launch_bounds__(256) void bc_table_kernel(AttnParams a, BcWs w) {
  __shared__ int base;
  const int bh = blockIdx.x;
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < bh; ++i) s += w.icnt[i];
    base = s;
    if (bh == (int)gridDim.x - 1) *w.nitems = s + w.icnt[bh];
  }
  __syncthreads();
  for (int blk = threadIdx.x; blk < w.nbk; blk += 256) {
    const int n = (w.tot[(int64_t)bh * w.nbk + blk] + w.rpi - 1) / w.rpi;
    const int o = base + w.ioff[(int64_t)bh * w.nbk + blk];
    for (int c = 0; c < n; ++c) {
      w.item_bk[o + c] = (uint32_t)(bh * w.nbk + blk);
      w.item_c[o + c] = (uint32_t)c;
    }
  }
}

__global__ __launch_bounds__(kBcRows) void bc_scatter_kernel(AttnParams a, BcWs w) {
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.G_sel + g;
  const int r = ch * kBcRows + threadIdx.x;
  if (r >= a.Nq) return;
  const int32_t* sel = a.sel + b * a.sels[0] + g * a.sels[1] + (int64_t)r * a.sels[2];
  const int32_t* rk = w.rank + ((int64_t)bh * a.Nq + r) * a.K;
  const int32_t* hg = w.hist + ((int64_t)bh * w.nch + ch) * w.nbk;
  uint32_t* lst = w.list + (int64_t)bh * a.Nq * a.K;
  if (a.K <= 16 && (a.K & 3) == 0) {
    // the row's list and ranks, then every slot's list base and chunk offset
    // loaded together (index clamped for slots that do not contribute)
    int blk[kBcListMax], vv[16], lb[16], ho[16];
    bc_load_list(a, sel, blk);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      int4 v4 = make_int4(-1, -1, -1, -1);
      if (4 * s4 < a.K) v4 = *(const int4*)(rk + 4 * s4);
      vv[4 * s4] = v4.x;
      vv[4 * s4 + 1] = v4.y;
      vv[4 * s4 + 2] = v4.z;
      vv[4 * s4 + 3] = v4.w;
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int bb = vv[s] >= 0 ? blk[s] : 0;
      lb[s] = w.lbase[(int64_t)bh * w.nbk + bb];
      ho[s] = hg[bb];
    }
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (vv[s] >= 0) lst[lb[s] + ho[s] + vv[s]] = (uint32_t)r | ((uint32_t)s << 24);
    return;
  }
  for (int s = 0; s < a.K; ++s) {
    const int v = rk[s];
    if (v < 0) continue;
    const int blk = sel[s * a.sels[3]];
    const int pos = w.lbase[(int64_t)bh * w.nbk + blk] + hg[blk] + v;
    lst[pos] = (uint32_t)r | ((uint32_t)s << 24);
  }
}

struct BcSmem {
  uint16_t ks[64 * kBcKs];
  uint16_t vt[64 * 128];    // V tile row-major, XOR-swizzled 16-byte chunks
};

// One work item: up to rpi = 64 / hpg rows that chose block blk of (request,
// group) bg, for each of the group's hpg query heads: MFMA row q = 16 wv + c16
// (wave wv, lane column c16) is row q / hpg of the item, head q % hpg.
__global__ __launch_bounds__(256) void bc_attn_kernel(AttnParams a, BcWs w, int xper) {
  // the items of one block are consecutive, and each XCD takes a run of
  // items: a block's keys staged by its items come from one XCD's L2
  const int item = xcd_item(blockIdx.x, xper);
  if (item >= *w.nitems) return;
  __shared__ __attribute__((aligned(16))) BcSmem sm;
  const uint32_t bk = w.item_bk[item];
  const int c = (int)w.item_c[item];
  const int bg = bk / w.nbk, blk = bk % w.nbk;
  const int b = bg / a.G_sel, g = bg % a.G_sel;
  const int kvh = (g * w.hpg) / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qq = lane >> 4, c16 = lane & 15;
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int nrow = min(w.rpi, w.tot[bk] - w.rpi * c);
  const uint32_t* lst = w.list + (int64_t)bg * a.Nq * a.K + w.lbase[bk] + w.rpi * c;

  // this lane's (row, head)
  const int qi = 16 * wid + c16;
  const int ri = qi / w.hpg;
  const int h = g * w.hpg + qi % w.hpg;
  const bool rvalid = ri < nrow;
  const uint32_t ent = rvalid ? lst[ri] : 0u;
  const int r = (int)(ent & 0xFFFFFFu);
  const int p = L - a.Nq + r;
  const int wstart = p - a.window + 1;
  bf16x8 Qb[4];
  if (rvalid) {
    const uint16_t* qp = (const uint16_t*)a.q.p + b * a.q.s[0] + h * a.q.s[1] + (int64_t)r * a.q.s[2] + 32 * qq;
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s] = *(const bf16x8*)(qp + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s] = (bf16x8){};
  }
  const float cs = a.scale * kBcLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.s[0] + kvh * a.k.s[1];
  const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.s[0] + kvh * a.v.s[1];
  const int klo = blk * a.bs, khi = min(klo + a.bs, L);   // keys [klo, khi) of the block

  for (int j0 = klo; j0 < khi; j0 += 64) {
    // stage 64 keys: chunk cc = tid + 256u -> key cc/16, 16-byte column cc%16
    u32x4 pk[4], pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = tid + 256 * u;
      int j = j0 + (cc >> 4);
      j = j < khi ? j : khi - 1;
      pk[u] = *(const u32x4*)(kbase + (int64_t)j * a.k.s[2] + 8 * (cc & 15));
      pv[u] = *(const u32x4*)(vbase + (int64_t)j * a.v.s[2] + 8 * (cc & 15));
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = tid + 256 * u;
      const int key = cc >> 4, col = cc & 15;
      *(u32x4*)&sm.ks[key * kBcKs + 8 * col] = pk[u];
      // V row-major, 16-byte chunk col of row key at col ^ (key mod 16)
      *(u32x4*)&sm.vt[key * 128 + 8 * (col ^ (key & 15))] = pv[u];
    }
    __syncthreads();
    if (__ballot(rvalid)) {
      f32x4 S[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        S[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const uint16_t* kr = &sm.ks[(16 * st + c16) * kBcKs + 32 * qq];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kr + 8 * s), Qb[s], S[st], 0, 0, 0);
      }
      // lane's keys j = j0 + 16 st + 4 qq + v for its row (column c16): in the
      // block, at or before the row, before its window
      float z[16];
      float tm = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = j0 + 16 * st + 4 * qq + v;
          const bool vis = rvalid && j < khi && j <= p && j < wstart;
          const float zz = vis ? S[st][v] * cs : -INFINITY;
          z[4 * st + v] = zz;
          tm = fmaxf(tm, zz);
        }
      tm = rows4_max(tm);
      const float mn = fmaxf(m, tm);
      float alpha = 1.f, ps = 0.f;
      if (mn > -INFINITY) {
        alpha = exp2f(m - mn);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          z[i] = exp2f(z[i] - mn);
          ps += z[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
      }
      ps = rows4_sum(ps);
      l = l * alpha + ps;
      m = mn;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
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
      // O += P V, two halves of 32 keys; k = 8 qq + v <-> keys 4 qq + v (v < 4), 16 + 4 qq + (v - 4)
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
        }
      }
    }
  }

  // partial of each row: lane holds dims 16 nt + c16 of rows 4 qq + v of
  // this wave; O / l in 16-bit fixed point against the row's largest |O / l|
  // (a maximum over the 16 lanes of the lane's DPP row), then m, l, scale
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = 4 * qq + v;                   // MFMA row within the wave (lane column rr holds its state)
    const float lr = __shfl(l, rr, 64);
    const float mr = __shfl(m, rr, 64);
    const uint32_t er = (uint32_t)__shfl((int)ent, rr, 64);
    const int hr = __shfl(h, rr, 64);
    const float il = lr > 0.f ? 1.0f / lr : 0.f;
    float on[8], mx = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      on[nt] = O[nt][v] * il;
      mx = fmaxf(mx, fabsf(on[nt]));
    }
    mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0x128, 0xf, 0xf, false)));
    mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0x124, 0xf, 0xf, false)));
    mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0x122, 0xf, 0xf, false)));
    mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0x121, 0xf, 0xf, false)));
    if ((16 * wid + rr) / w.hpg >= nrow) continue;
    const int rw = (int)(er & 0xFFFFFFu), sw = (int)(er >> 24);
    float* pp = w.part + ((((int64_t)b * a.Hq + hr) * a.Nq + rw) * a.K + sw) * kBcPart;
    const float sc = mx > 0.f ? mx : 1.f;
    const float qs = 32767.0f / sc;
    int16_t* pq = (int16_t*)(pp + 4);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) pq[16 * nt + c16] = (int16_t)__float2int_rn(fminf(fmaxf(on[nt] * qs, -32767.f), 32767.f));
    if (c16 == 0) *(f32x4*)pp = (f32x4){mr, lr, sc, 0.f};
  }
}

// per row (16 threads, 16 rows per workgroup): merge the window part (O
// normalized, LSE) with the block partials. Thread part of a row loads the
// header (m, l, scale) and the rank of slots part, part + 16, ... into LDS;
// then each thread takes 8 dims of every slot with one 16-byte load per
// slot, all of a row's slots in flight together.
constexpr int kBcCombRows = 16;
__global__ __launch_bounds__(256) void bc_combine_kernel(AttnParams a, BcWs w) {
  __shared__ float sm_m[kBcCombRows][256], sm_w[kBcCombRows][256], sm_s[kBcCombRows][256];
  const int rl = threadIdx.x >> 4, part = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * kBcCombRows + rl;
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Nq;
  const bool live = row < nrows;
  const int K = a.K;
  // the row's group list ranks: row = ((b Hq + h) Nq + r), group g = h / hpg
  const int64_t grow = live ? ((row / a.Nq / a.Hq) * a.G_sel + (row / a.Nq % a.Hq) / w.hpg) * a.Nq + row % a.Nq : 0;
  const float lw = live ? w.lse_w[row] : -INFINITY;   // with the headers: one round of loads
  if (live)
    for (int s = part; s < K; s += 16) {
      // rank and header loaded together (a header of a slot that does not
      // contribute is read but not used)
      const int rk = w.rank[grow * K + s];
      const f32x4 hd = *(const f32x4*)(w.part + (row * K + s) * kBcPart);
      const bool c = rk >= 0;
      const float ms = c ? hd[0] : -INFINITY, ls = c ? hd[1] : 0.f, ss = c ? hd[2] * (1.0f / 32767.0f) : 0.f;
      sm_m[rl][s] = ms;
      sm_w[rl][s] = ls;              // l, then the weight once M is known
      sm_s[rl][s] = ss;              // scale / 32767
    }
  __syncthreads();
  if (!live) return;
  const int r = (int)(row % a.Nq), bh = (int)(row / a.Nq);
  const int h = bh % a.Hq, b = bh / a.Hq;
  float* o = a.o + b * a.os[0] + h * a.os[1] + (int64_t)r * a.os[2] + 8 * part;
  // window part as (m, l, O) in base-2 units: m = LSE / ln 2, l = 1, O normalized
  const float mw = lw > -INFINITY ? lw * kBcLog2e : -INFINITY;
  float M = mw;
  for (int s = 0; s < K; ++s) M = fmaxf(M, sm_m[rl][s]);
  float Ls = 0.f, Os[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M > -INFINITY) {
    // a partial holds O / l: its weight is l e^(m - M); every slot's values
    // are loaded (an int16 is always finite; a slot that does not contribute
    // gets weight 0), and the window part's output after the first slots'
    const char* base = (const char*)(w.part + row * K * kBcPart + 4) + 16 * part;
    for (int s0 = 0; s0 < K; s0 += 16) {
      u32x4 x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = *(const u32x4*)(base + (int64_t)min(s0 + u, K - 1) * (4 * kBcPart));
      if (s0 == 0) {
        float ov[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = o[e];
        const float f = mw > -INFINITY ? exp2f(mw - M) : 0.f;
        Ls = f;
#pragma unroll
        for (int e = 0; e < 8; ++e) Os[e] = f > 0.f ? ov[e] * f : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int s = s0 + u;
        const bool c = s < K && sm_m[rl][s < K ? s : 0] > -INFINITY;
        const float f = c ? exp2f(sm_m[rl][s] - M) * sm_w[rl][s] : 0.f;
        const float fs = c ? f * sm_s[rl][s] : 0.f;
        Ls += f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Os[2 * e] += (float)(int16_t)(x[u][e] & 0xFFFFu) * fs;
          Os[2 * e + 1] += (float)(int16_t)(x[u][e] >> 16) * fs;
        }
      }
    }
  }
  const float il = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = Os[e] * il;
  if (a.lse && part == 0) a.lse[row] = Ls > 0.f ? (M + log2f(Ls)) * kBcLn2 : -INFINITY;
}

hipError_t launch_attn_blocks(const AttnParams& a0, hipStream_t st) {
  AttnParams a = a0;
  size_t need = 0;
  BcWs w = bc_layout(a, a.ws, &need);
  const dim3 gc(w.nch, a.G_sel, a.B);
  const int bh = a.B * a.Hq;
  const int bg = a.B * a.G_sel;
  hipLaunchKernelGGL(bc_count_kernel, gc, dim3(kBcRows), 0, st, a, w);
  hipLaunchKernelGGL(bc_scan_kernel, dim3(bg), dim3(256), 0, st, a, w);
  hipLaunchKernelGGL(bc_table_kernel, dim3(bg), dim3(256), 0, st, a, w);
  hipLaunchKernelGGL(bc_scatter_kernel, gc, dim3(kBcRows), 0, st, a, w);
  const int per = (w.maxitems + 7) / 8;
  hipLaunchKernelGGL(bc_attn_kernel, dim3(8 * per), dim3(256), 0, st, a, w, per);
  // window part: the tiled kernel, its LSE into the workspace
  AttnParams aw = a;
  aw.mode = 2;
  aw.n_global = 0;
  aw.lse = w.lse_w;
  hipError_t e = launch_attn_tile(aw, st);
  if (e != hipSuccess) return e;
  const int64_t nrows = (int64_t)bh * a.Nq;
  hipLaunchKernelGGL(bc_combine_kernel, dim3((unsigned)((nrows + kBcCombRows - 1) / kBcCombRows)), dim3(256), 0, st, a,
                     w);
  return hipGetLastError();
}

}  // namespace sp
