// Three-branch NSA attention ("Sparse Attention in 2026", NSA paragraph;
// "Sparse Attention" (completesystemdesign.dev), three parallel paths):
//
//  * compression: the K and V rows of every complete block are mean-pooled
//    into one entry (nsa_pool: the mean formed in float64, then kept as a
//    pair of bf16 parts hi + lo for the MFMA tile kernel, about 2^-17 of the
//    mean, or rounded once to float32 for the generic kernel), and each query
//    attends over the entries of its complete past blocks (attention mode 5);
//  * selection: attention over the tokens of the blocks chosen by
//    spattn_block_select, whose scores are the compression branch's own
//    logits q . mean(k) (attention mode 3 without a window);
//  * window: attention over the last `window` keys (mode 2);
//
// each branch with its own softmax, then o = g_cmp o_cmp + g_sel o_sel +
// g_win o_win per (row, head) from the gate inputs (nsa_combine). A branch
// with no visible entry contributes 0.
#include "common.h"
#include "internal.h"

namespace sp {

// float64 -> bf16 bits, round to nearest even in one step (rounding through
// float32 first could round twice): the float64 pattern is rounded at bf16's
// last significand bit, after which it converts to float32 exactly.
SP_DEV uint32_t f64_to_bf16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;
  u = (u + ((1ull << 44) - 1ull) + lsb) & ~((1ull << 45) - 1ull);
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
}

// One workgroup per (block, KV head, request), one thread per dimension: the
// block's rows summed in float64 (exact for bf16/f32 rows spanning less than
// 2^39 in magnitude), divided by the power-of-two block size (exact), then
// written as hi = bf16(mean), lo = bf16(mean - hi) (kclo/vclo given) or as the
// nearest float32.
__global__ __launch_bounds__(128) void nsa_pool_kernel(AttnParams a, void* kc, void* vc, uint16_t* kclo,
                                                       uint16_t* vclo, int nbmax) {
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = min(a.ctx_len ? a.ctx_len[b] : a.ctx, a.ctx);
  const int c = threadIdx.x;
  if (blk >= L / a.bs || c >= a.d) return;
  const int64_t kb = b * a.k.s[0] + h * a.k.s[1] + (int64_t)blk * a.bs * a.k.s[2] + c;
  const int64_t vb = b * a.v.s[0] + h * a.v.s[1] + (int64_t)blk * a.bs * a.v.s[2] + c;
  double sk = 0.0, sv = 0.0;
  if (a.k.dt == DT_BF16) {
    const uint16_t* kp = (const uint16_t*)a.k.p;
    const uint16_t* vp = (const uint16_t*)a.v.p;
#pragma unroll 8
    for (int t = 0; t < a.bs; ++t) {
      sk += (double)bf16_to_f32(kp[kb + t * a.k.s[2]]);
      sv += (double)bf16_to_f32(vp[vb + t * a.v.s[2]]);
    }
  } else {
    const float* kp = (const float*)a.k.p;
    const float* vp = (const float*)a.v.p;
#pragma unroll 8
    for (int t = 0; t < a.bs; ++t) {
      sk += (double)kp[kb + t * a.k.s[2]];
      sv += (double)vp[vb + t * a.v.s[2]];
    }
  }
  const double inv = 1.0 / (double)a.bs;              // a power of two: exact
  const int64_t o = (((int64_t)b * a.Hkv + h) * nbmax + blk) * a.d + c;
  const double mk = sk * inv, mv = sv * inv;
  if (kclo) {
    const uint32_t hk = f64_to_bf16_rne(mk), hv = f64_to_bf16_rne(mv);
    ((uint16_t*)kc)[o] = (uint16_t)hk;
    ((uint16_t*)vc)[o] = (uint16_t)hv;
    kclo[o] = (uint16_t)f64_to_bf16_rne(mk - (double)bf16_to_f32(hk));   // exact difference
    vclo[o] = (uint16_t)f64_to_bf16_rne(mv - (double)bf16_to_f32(hv));
  } else {
    ((float*)kc)[o] = (float)mk;
    ((float*)vc)[o] = (float)mv;
  }
}

// One workgroup per (request, head, row), one thread per dimension.
__global__ __launch_bounds__(128) void nsa_combine_kernel(NsaParams p, const float* oc, const float* osel,
                                                          const float* ow) {
  const AttnParams& a = p.a;
  const int row = blockIdx.x;
  const int r = row % a.Nq, h = (row / a.Nq) % a.Hq, b = row / (a.Nq * a.Hq);
  const int c = threadIdx.x;
  if (c >= a.d) return;
  const float* g = p.gates + b * p.gs[0] + h * p.gs[1] + r * p.gs[2];
  const int64_t i = (int64_t)row * a.d + c;
  float o = g[0] * oc[i];
  o = fmaf(g[p.gs[3]], osel[i], o);
  o = fmaf(g[2 * p.gs[3]], ow[i], o);
  p.o[b * p.os[0] + h * p.os[1] + r * p.os[2] + c] = o;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// The three branches' attention parameters, with the workspace laid out as
// pooled K | pooled V | (split: K low parts | V low parts) | O of each branch
// [B, Hq, Nq, d] f32 | branch workspace.
struct NsaLayout {
  AttnParams cmp, sel, win;
  size_t kc, vc, kclo, vclo, oc, os, ow, attn, total;
  int nbmax;
  bool split;              // bf16 hi/lo entries on the tile kernel, else float32 entries
};

static NsaLayout nsa_layout(const NsaParams& p) {
  NsaLayout l;
  const AttnParams& a = p.a;
  l.nbmax = a.ctx / a.bs;
  l.cmp = a;
  l.cmp.mode = 5;
  for (View4* vw : {&l.cmp.k, &l.cmp.v}) {
    vw->n[2] = l.nbmax;
    vw->s[3] = 1;
    vw->s[2] = a.d;
    vw->s[1] = (int64_t)l.nbmax * a.d;
    vw->s[0] = (int64_t)a.Hkv * l.nbmax * a.d;
  }
  l.split = a.k.dt == DT_BF16 && attn_tile_ok(l.cmp);
  if (!l.split) l.cmp.k.dt = l.cmp.v.dt = DT_F32;
  const size_t pooled = (size_t)a.B * a.Hkv * l.nbmax * a.d * (l.split ? 2 : 4);
  const size_t obytes = (size_t)a.B * a.Hq * a.Nq * a.d * sizeof(float);
  size_t off = 0;
  l.kc = off;
  off += al256(pooled);
  l.vc = off;
  off += al256(pooled);
  l.kclo = l.vclo = 0;
  if (l.split) {
    l.kclo = off;
    off += al256(pooled);
    l.vclo = off;
    off += al256(pooled);
  }
  l.oc = off;
  off += al256(obytes);
  l.os = off;
  off += al256(obytes);
  l.ow = off;
  off += al256(obytes);
  l.attn = off;
  auto dense_out = [&](AttnParams& x) {
    x.os[3] = 1;
    x.os[2] = a.d;
    x.os[1] = (int64_t)a.Nq * a.d;
    x.os[0] = (int64_t)a.Hq * a.Nq * a.d;
    x.lse = nullptr;
  };
  dense_out(l.cmp);
  l.sel = a;
  l.sel.mode = 3;
  l.sel.window = 0;
  dense_out(l.sel);
  l.win = a;
  l.win.mode = 2;
  l.win.n_global = 0;
  l.win.stride = 0;
  dense_out(l.win);
  size_t aw = attn_ws_bytes(l.cmp);
  aw = aw > attn_ws_bytes(l.sel) ? aw : attn_ws_bytes(l.sel);
  aw = aw > attn_ws_bytes(l.win) ? aw : attn_ws_bytes(l.win);
  l.total = off + aw;
  return l;
}

size_t nsa_ws_bytes(const NsaParams& p) { return nsa_layout(p).total; }

hipError_t launch_nsa(const NsaParams& p, hipStream_t st) {
  NsaLayout l = nsa_layout(p);
  char* w = (char*)p.ws;
  const AttnParams& a = p.a;
  void* kc = w + l.kc;
  void* vc = w + l.vc;
  float* oc = (float*)(w + l.oc);
  float* osel = (float*)(w + l.os);
  float* ow = (float*)(w + l.ow);
  hipError_t e;
  uint16_t* kclo = l.split ? (uint16_t*)(w + l.kclo) : nullptr;
  uint16_t* vclo = l.split ? (uint16_t*)(w + l.vclo) : nullptr;
  if (l.nbmax > 0) {
    hipLaunchKernelGGL(nsa_pool_kernel, dim3(l.nbmax, a.Hkv, a.B), dim3(128), 0, st, a, kc, vc, kclo, vclo,
                       l.nbmax);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  l.cmp.k.p = kc;
  l.cmp.v.p = vc;
  l.cmp.klo = kclo;
  l.cmp.vlo = vclo;
  l.cmp.o = oc;
  l.sel.o = osel;
  l.win.o = ow;
  for (AttnParams* x : {&l.cmp, &l.sel, &l.win}) {
    x->ws = w + l.attn;
    x->ws_bytes = l.total - l.attn;
    if ((e = launch_attention(*x, st)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(nsa_combine_kernel, dim3(a.B * a.Hq * a.Nq), dim3(128), 0, st, p, (const float*)oc,
                     (const float*)osel, (const float*)ow);
  return hipGetLastError();
}

}  // namespace sp
