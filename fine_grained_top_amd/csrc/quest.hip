// Query-aware page selection without a trained indexer ("Sparse Attention"
// (completesystemdesign.dev), inference-only alternatives: Quest-style
// page-wise KV selection; the criterion is Quest's (Tang et al., 2024)).
//
// Each complete page keeps, per KV head and channel, the smallest and the
// largest key among its tokens (quest_bounds: exact in the key dtype). For a
// query row q of selection group g (the query heads that share one page list)
// a page's key is the float32 nearest to
//     U = sum over the group's heads h, channels c of max(q_hc m_c, q_hc M_c),
// the largest value q . x takes over the box [m, M], so no token of the page
// scores above it. The products are exact in float64 (bf16 and float32
// operands), their sum is taken in float64 and certified against a rigorous
// rounding bound; for a page within the bound of a float32 rounding boundary
// the sum is redone with every addition checked for rounding, and only if one
// rounded is it summed exactly in a wide fixed-point accumulator. The n_local
// recent pages are always read; the others are ranked by (key descending,
// page ascending) by the page-selection kernel.
#include "common.h"
#include "exact.h"
#include "internal.h"

namespace sp {

constexpr int kQkPages = 64;      // pages per key workgroup (16 quarter-waves, 4 pages each)
constexpr int kQkMaxHeads = 16;   // query heads per selection group

// One workgroup per (complete page, KV head, request), one thread per channel.
__global__ __launch_bounds__(128) void quest_bounds_kernel(QuestParams p) {
  const int pg = blockIdx.x, h = blockIdx.y, b = blockIdx.z, c = threadIdx.x;
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  if (pg >= (L >> p.lgP) || c >= p.d) return;
  const int64_t pp = p.ptab[b * p.pts[0] + pg * p.pts[1]];
  const int64_t base = pp * p.kp.s[0] + h * p.kp.s[1] + c;
  const int P = 1 << p.lgP;
  const int64_t o = b * p.bs[0] + pg * p.bs[1] + h * p.bs[2] + c;
  if (p.kp.dt == DT_BF16) {
    const uint16_t* k = (const uint16_t*)p.kp.p;
    float mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < P; ++t) {
      const float x = bf16_to_f32(k[base + t * p.kp.s[2]]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    uint16_t* dst = (uint16_t*)p.bnd;
    dst[o] = (uint16_t)(__float_as_uint(mn) >> 16);      // bf16 values: the low half is zero
    dst[o + p.d] = (uint16_t)(__float_as_uint(mx) >> 16);
  } else {
    const float* k = (const float*)p.kp.p;
    float mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < P; ++t) {
      const float x = k[base + t * p.kp.s[2]];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    float* dst = (float*)p.bnd;
    dst[o] = mn;
    dst[o + p.d] = mx;
  }
}

// Exact key of one page by one lane: each term's larger product chosen by an
// exact comparison and summed in the wide accumulator.
SP_DEV float quest_exact_key(const QuestParams& p, const float* qs, int hg, int64_t bo) {
  DotAcc acc;
  acc.clear();
  for (int h = 0; h < hg; ++h)
    for (int c = 0; c < p.d; ++c) {
      const double qv = (double)qs[h * p.d + c];
      const double mn = load_f64(p.bnd, p.dt, bo + c), mx = load_f64(p.bnd, p.dt, bo + p.d + c);
      const double bsel = qv * mx >= qv * mn ? mx : mn;
      int64_t mq, mb;
      int eq, eb;
      bool nq, nb;
      split24(qv, mq, eq, nq);
      split24(bsel, mb, eb, nb);
      if (mq == 0 || mb == 0) continue;
      acc.add((uint64_t)mq * (uint64_t)mb, eq + eb - kDotBase, nq != nb);
    }
  return wide_to_f32(acc, kDotBase);
}

// Keys of the candidate pages of one row, pages [blockIdx.x * kQkPages, ...),
// written as order keys to pkg[row * npmax + page]; 16 lanes per page, each
// lane d/16 channels of every head of the group.
__global__ __launch_bounds__(256) void quest_keys_kernel(QuestParams p, uint32_t* pkg, int npmax) {
  __shared__ float qs[kQkMaxHeads * 128];
  const PageSelParams& s = p.sel;
  const int G = s.t.G;
  const int row = blockIdx.y;
  const int r = row % p.Nq, g = (row / p.Nq) % G, b = row / (p.Nq * G);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  if (pos < 0) return;
  const int npc = max(0, (pos >> p.lgP) + 1 - s.n_local);
  if (npc <= s.t.K || s.t.K == 0) return;           // the selection kernel needs no keys for this row
  const int pg0 = blockIdx.x * kQkPages;
  if (pg0 >= npc) return;
  const int pg1 = min(pg0 + kQkPages, npc);
  const int hg = p.Hq / G, h0 = g * hg, kvh = h0 / (p.Hq / p.Hkv);
  for (int e = threadIdx.x; e < hg * p.d; e += 256) {
    const int h = e / p.d, c = e - h * p.d;
    qs[e] = (float)load_f64(p.q.p, p.q.dt, b * p.q.s[0] + (h0 + h) * p.q.s[1] + r * p.q.s[2] + c);
  }
  __syncthreads();
  const int sub = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int cpl = p.d >> 4;                          // channels per lane: 4 or 8
  const int c0 = sub * cpl;
  const double n_terms = (double)(hg * p.d + 16);
  for (int it = pg0; it < pg1; it += 16) {           // uniform trip count: whole waves take the shuffles
    const int pg = it + grp;
    const bool act = pg < pg1;
    const int64_t bo = b * p.bs[0] + (int64_t)(act ? pg : pg0) * p.bs[1] + kvh * p.bs[2];
    float mn[8], mx[8];
    if (p.dt == DT_BF16) {
      const uint16_t* bp = (const uint16_t*)p.bnd + bo + c0;
      if (cpl == 8) {
        const u32x4 a = *(const u32x4*)bp, z = *(const u32x4*)(bp + p.d);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          mn[2 * u] = bf16_to_f32(a[u] & 0xFFFFu);
          mn[2 * u + 1] = bf16_to_f32(a[u] >> 16);
          mx[2 * u] = bf16_to_f32(z[u] & 0xFFFFu);
          mx[2 * u + 1] = bf16_to_f32(z[u] >> 16);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          mn[u] = bf16_to_f32(bp[u]);
          mx[u] = bf16_to_f32(bp[p.d + u]);
        }
      }
    } else {
      const float* bp = (const float*)p.bnd + bo + c0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < cpl) {
          mn[u] = bp[u];
          mx[u] = bp[p.d + u];
        }
      }
    }
    // max(q m, q M) = q (q >= 0 ? M : m) since m <= M: one exact product per
    // term, added with a single rounding by the fma
    double y = 0.0, A = 0.0;
    for (int h = 0; h < hg; ++h) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < cpl) {
          const float qf = qs[h * p.d + c0 + u];
          const double qv = (double)qf, bv = (double)(qf >= 0.f ? mx[u] : mn[u]);
          y = fma(qv, bv, y);
          A = fma(fabs(qv), fabs(bv), A);
        }
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {               // the 16 lanes of the page
      y += __shfl_xor(y, o, 64);
      A += __shfl_xor(A, o, 64);
    }
    // recursive and pairwise sums of n terms err by at most (n - 1) 2^-53 sum|t|
    float key;
    if (!certify(y, n_terms * 2.220446049250313e-16 * A, key)) {
      // near a float32 rounding boundary (the same for the page's 16 lanes): the
      // sum again with every addition checked (TwoSum); bf16 products are short,
      // so the float64 sum is usually exact and rounds once
      double ys = 0.0, As = 0.0;
      bool ex = true;
      for (int h = 0; h < hg; ++h) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (u < cpl) {
            const float qf = qs[h * p.d + c0 + u];
            const double t = (double)qf * (double)(qf >= 0.f ? mx[u] : mn[u]);   // exact
            xadd(ys, ex, t);
            As += fabs(t);
          }
        }
      }
      group_xreduce<16>(ys, ex, As);
      if (ex) key = (float)ys + 0.0f;
      else if (sub == 0) key = quest_exact_key(p, qs, hg, bo);
    }
    if (act && sub == 0) pkg[(int64_t)row * npmax + pg] = f32_order_key(key);
  }
}

size_t quest_ws_bytes(const QuestParams& p) {
  return (size_t)p.B * p.sel.t.G * p.Nq * p.maxp * sizeof(uint32_t);
}

hipError_t launch_quest_bounds(const QuestParams& p, hipStream_t st) {
  hipLaunchKernelGGL(quest_bounds_kernel, dim3(p.maxp, p.Hkv, p.B), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_quest_select(const QuestParams& p, hipStream_t st) {
  const int rows = p.B * p.sel.t.G * p.Nq;
  uint32_t* pkg = (uint32_t*)p.sel.ws;
  hipLaunchKernelGGL(quest_keys_kernel, dim3((p.maxp + kQkPages - 1) / kQkPages, rows), dim3(256), 0, st, p, pkg,
                     p.maxp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_page_select_keys(p.sel, pkg, p.maxp, st);
}

}  // namespace sp
