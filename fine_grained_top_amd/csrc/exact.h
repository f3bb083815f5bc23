// Exact selection keys on the device.
//
// A selection key is the float32 nearest (ties to even) to the exact real
// value of a score: a dot product q.k, a ReLU-gated weighted sum of such dot
// products over indexer heads, or the mean over a block of keys of q.k. The
// key does not depend on summation order, so index sets chosen on it are
// reproducible bit for bit on any machine.
//
// Evaluation: float64 with a rigorous error bound first (products of inputs
// with <= 24-bit significands are exact in float64; an n-term float64 sum in
// any order is within n * 2^-53 * sum|terms| of the exact sum). When the whole
// error interval rounds to one float32 that value is the key. Alongside, every
// float64 addition is checked with an error-free transformation (TwoSum;
// TwoProduct by fma for products that need not be exact): when no addition
// rounded, the float64 result is the exact value and one float32 rounding
// gives the key, also when it sits exactly on a rounding boundary (common
// for bf16 data, whose sums are short). Otherwise (the exact value sits next
// to a float32 rounding boundary) the sum is formed exactly in a wide two's-
// complement fixed-point accumulator and rounded by hand. Input significands
// are at most 24 bits, exponents within float32's.
#pragma once
#include "common.h"
#include "internal.h"

namespace sp {

// s += t with exactness tracking: exact stays true while no addition rounded
// (TwoSum recovers the rounding error of s + t exactly).
SP_DEV void xadd(double& s, bool& exact, double t) {
#pragma clang fp contract(off)
  const double n = s + t;
  const double bb = n - s;
  const double err = (s - (n - bb)) + (t - bb);
  exact = exact && err == 0.0;
  s = n;
}

// s += a * b exactly tracked: the product's rounding error (fma) is added too.
SP_DEV void xadd_prod(double& s, bool& exact, double a, double b) {
#pragma clang fp contract(off)
  const double p = a * b;
  const double pe = fma(a, b, -p);
  xadd(s, exact, p);
  if (pe != 0.0) xadd(s, exact, pe);
}

// All-reduce of a tracked sum and of its magnitude sum over a group of W
// aligned lanes (W = 64: the wave; 32: a half-wave); the butterfly gives every
// lane of the group the same value, and exact becomes group-uniform.
template <int W>
SP_DEV void group_xreduce(double& y, bool& exact, double& A) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) {
    xadd(y, exact, __shfl_xor(y, o, 64));
    A += __shfl_xor(A, o, 64);
  }
  const uint64_t bad = ballot(!exact);
  const int base = (threadIdx.x & 63) & ~(W - 1);
  const uint64_t gm = W == 64 ? ~0ull : ((1ull << W) - 1) << base;
  exact = (bad & gm) == 0;
}

// A float64 rotated by N lanes within each 16-lane row (DPP row_ror; every
// source lane is valid).
template <int N>
SP_DEV double row_ror_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x120 + N, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x120 + N, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// group_xreduce<16> of NH independent sums at once: rotations by 8, 4, 2, 1
// within the 16-lane row, the sums interleaved level by level. Lanes add the
// same pairs in swapped order (commutative, so every lane ends with the same
// bits, and both see the same rounding).
template <int NH>
SP_DEV void row16_xreduce(double (&y)[NH], bool (&exact)[NH], double (&A)[NH]) {
#define SP_ROR_STEP(N)                                   \
  _Pragma("unroll") for (int u = 0; u < NH; ++u) {       \
    xadd(y[u], exact[u], row_ror_f64<N>(y[u]));          \
    A[u] += row_ror_f64<N>(A[u]);                        \
  }
  SP_ROR_STEP(8)
  SP_ROR_STEP(4)
  SP_ROR_STEP(2)
  SP_ROR_STEP(1)
#undef SP_ROR_STEP
  const uint64_t gm = 0xFFFFull << ((threadIdx.x & 63) & ~15);
#pragma unroll
  for (int u = 0; u < NH; ++u) exact[u] = (ballot(!exact[u]) & gm) == 0;
}
SP_DEV void wave_xreduce(double& y, bool& exact, double& A) { group_xreduce<64>(y, exact, A); }

// float32 key of an exact float64 value (-0 read as +0)
SP_DEV float key_of_exact(double y) { return (float)y + 0.0f; }

SP_DEV double load_f64(const void* p, int dtype, int64_t i) {
  if (dtype == DT_F32) return (double)((const float*)p)[i];
  if (dtype == DT_BF16) return (double)bf16_to_f32(((const uint16_t*)p)[i]);
  return (double)fp8_to_f32(((const uint8_t*)p)[i]);
}

// out[e] = element i + e of a row of type dtype as float64 (exact), 0 from
// element i + avail on. A whole run of four is one vector load: rows start
// 16-byte aligned and i is a multiple of four, so the run is aligned to its
// own size.
template <int N>
SP_DEV void load_run_f64(const void* p, int dtype, int64_t i, int avail, double (&out)[N]) {
  if constexpr (N == 4) {
    if (avail >= 4) {
      if (dtype == DT_FP8) {
        const uint32_t w = *(const uint32_t*)((const uint8_t*)p + i);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        out[0] = lo[0];
        out[1] = lo[1];
        out[2] = hi[0];
        out[3] = hi[1];
      } else if (dtype == DT_BF16) {
        const u32x2 w = *(const u32x2*)((const uint16_t*)p + i);
        out[0] = bf16_to_f32(w[0] & 0xFFFFu);
        out[1] = bf16_to_f32(w[0] >> 16);
        out[2] = bf16_to_f32(w[1] & 0xFFFFu);
        out[3] = bf16_to_f32(w[1] >> 16);
      } else {
        const f32x4 w = *(const f32x4*)((const float*)p + i);
        out[0] = w[0];
        out[1] = w[1];
        out[2] = w[2];
        out[3] = w[3];
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < N; ++e) out[e] = e < avail ? load_f64(p, dtype, i + e) : 0.0;
}

// value = m * 2^e with m an integer of at most 24 bits (exact for our formats).
SP_DEV void split24(double v, int64_t& m, int& e, bool& neg) {
  neg = v < 0;
  double a = neg ? -v : v;
  if (a == 0.0) { m = 0; e = 0; return; }
  int ex;
  double f = frexp(a, &ex);                 // a = f * 2^ex, f in [0.5, 1)
  m = (int64_t)ldexp(f, 24);
  e = ex - 24;
}

// Wide accumulator: NL little-endian 32-bit limbs, two's complement, value =
// sum(limb_i * 2^(32 i)) * 2^BASE.
template <int NL>
struct WideAcc {
  uint32_t l[NL];
  SP_DEV void clear() {
    for (int i = 0; i < NL; ++i) l[i] = 0;
  }
  // add (neg ? -1 : 1) * m * 2^bit, m < 2^57, bit >= 0
  SP_DEV void add(uint64_t m, int bit, bool neg) {
    if (m == 0) return;
    int li = bit >> 5, sh = bit & 31;
    uint32_t p[3];
    p[0] = (uint32_t)(m << sh);
    p[1] = sh ? (uint32_t)(m >> (32 - sh)) : (uint32_t)(m >> 32);
    p[2] = sh ? (uint32_t)(m >> (64 - sh)) : 0u;
    if (!neg) {
      uint64_t c = 0;
      for (int i = li; i < NL; ++i) {
        uint64_t s = (uint64_t)l[i] + c + (i - li < 3 ? p[i - li] : 0u);
        l[i] = (uint32_t)s;
        c = s >> 32;
        if (i - li >= 2 && c == 0) break;
      }
    } else {
      int64_t br = 0;
      for (int i = li; i < NL; ++i) {
        int64_t s = (int64_t)l[i] - br - (int64_t)(i - li < 3 ? p[i - li] : 0u);
        br = s < 0 ? 1 : 0;
        l[i] = (uint32_t)s;
        if (i - li >= 2 && br == 0) break;
      }
    }
  }
  SP_DEV bool negative() const { return (l[NL - 1] >> 31) != 0; }
  SP_DEV bool zero() const {
    for (int i = 0; i < NL; ++i)
      if (l[i]) return false;
    return true;
  }
  SP_DEV void negate() {
    uint64_t c = 1;
    for (int i = 0; i < NL; ++i) {
      uint64_t s = (uint64_t)(~l[i]) + c;
      l[i] = (uint32_t)s;
      c = s >> 32;
    }
  }
  SP_DEV int top_bit() const {
    for (int i = NL - 1; i >= 0; --i)
      if (l[i]) return 32 * i + 31 - __builtin_clz(l[i]);
    return -1;
  }
  SP_DEV uint32_t bit(int b) const { return b < 0 ? 0u : (l[b >> 5] >> (b & 31)) & 1u; }
  SP_DEV bool any_below(int b) const {   // any set bit at index < b
    if (b <= 0) return false;
    int li = b >> 5, sh = b & 31;
    for (int i = 0; i < li; ++i)
      if (l[i]) return true;
    return sh ? (l[li] & ((1u << sh) - 1u)) != 0 : false;
  }
  SP_DEV uint32_t bits(int lo, int n) const {  // n <= 25 bits starting at lo (lo >= 0)
    uint32_t r = 0;
    for (int k = 0; k < n; ++k) r |= bit(lo + k) << k;
    return r;
  }
};

// Round (acc * 2^(base)) to the nearest float32, ties to even.
template <int NL>
SP_DEV float wide_to_f32(WideAcc<NL> acc, int base) {
  bool neg = acc.negative();
  if (neg) acc.negate();
  int P = acc.top_bit();
  if (P < 0) return 0.0f;
  int E = P + base;
  if (E > 127) return neg ? -INFINITY : INFINITY;
  int qexp = (E > -126 ? E : -126) - 23;
  int qb = qexp - base;               // bit index of the float32 ulp
  uint32_t mant;
  bool guard, sticky;
  if (qb <= 0) {                       // every bit is kept
    mant = acc.bits(0, P + 1) << (-qb);
    guard = false;
    sticky = false;
  } else {
    mant = acc.bits(qb, P - qb + 1);
    guard = acc.bit(qb - 1) != 0;
    sticky = acc.any_below(qb - 1);
  }
  if (guard && (sticky || (mant & 1u))) mant += 1u;
  float r = ldexpf((float)mant, qexp);
  return neg ? -r : r;
}

// Exact dot product sum_c q[c]*k[c] into an accumulator with base -352 (20 limbs).
constexpr int kDotBase = -352;
typedef WideAcc<20> DotAcc;
SP_DEV void exact_dot_acc(DotAcc& acc, const void* q, int qt, int64_t qoff, const void* k, int kt,
                          int64_t koff, int n) {
  for (int c = 0; c < n; ++c) {
    int64_t mq, mk;
    int eq, ek;
    bool nq, nk;
    split24(load_f64(q, qt, qoff + c), mq, eq, nq);
    split24(load_f64(k, kt, koff + c), mk, ek, nk);
    if (mq == 0 || mk == 0) continue;
    acc.add((uint64_t)mq * (uint64_t)mk, eq + ek - kDotBase, nq != nk);
  }
}

// ---------------------------------------------------------------- keys

struct IndexerRow {        // one query row of one selection group
  const void* q;           // q_idx row base: head h at q + h*qh_stride
  int qt;                  // dtype
  int64_t qh_stride;       // elements between heads
  const void* k;           // k_idx row base of key 0 for this group
  int kt;
  int64_t k_stride;        // elements between keys
  const float* w;          // weights of the group's heads (stride w_stride), may be null in DOT
  int64_t w_stride;
  int H;                   // heads in the group (1 in DOT)
  int d;                   // indexer head dim
  int relu;                // 1 = weighted ReLU, 0 = plain dot
};

// The indexer row of query row r of request b, selection group g.
SP_DEV IndexerRow indexer_row(const IndexerParams& x, int b, int g, int r) {
  IndexerRow ir;
  const int hpg = x.hpg;
  const int kg = x.G_k == 1 ? 0 : g;
  const int esz = x.q.dt == DT_F32 ? 4 : 2;
  const int ksz = x.k.dt == DT_F32 ? 4 : (x.k.dt == DT_BF16 ? 2 : 1);
  ir.q = (const char*)x.q.p + (b * x.q.s[0] + r * x.q.s[1] + (int64_t)g * hpg * x.q.s[2]) * esz;
  ir.qt = x.q.dt;
  ir.qh_stride = x.q.s[2];
  ir.k = (const char*)x.k.p + (b * x.k.s[0] + kg * x.k.s[2]) * ksz;
  ir.kt = x.k.dt;
  ir.k_stride = x.k.s[1];
  ir.w = x.relu ? x.w + b * x.ws_[0] + r * x.ws_[1] + (int64_t)g * hpg * x.ws_[2] : nullptr;
  ir.w_stride = x.ws_[2];
  ir.H = hpg;
  ir.d = x.d_I;
  ir.relu = x.relu;
  return ir;
}

SP_DEV float exact_key_slow(const IndexerRow& r, int64_t j) {
  int64_t koff = j * r.k_stride;
  if (!r.relu) {
    DotAcc acc;
    acc.clear();
    exact_dot_acc(acc, r.q, r.qt, 0, r.k, r.kt, koff, r.d);
    return wide_to_f32(acc, kDotBase);
  }
  WideAcc<30> tot;   // base -544
  tot.clear();
  for (int h = 0; h < r.H; ++h) {
    DotAcc acc;
    acc.clear();
    exact_dot_acc(acc, r.q, r.qt, h * r.qh_stride, r.k, r.kt, koff, r.d);
    if (acc.negative() || acc.zero()) continue;      // ReLU
    int64_t mw;
    int ew;
    bool nw;
    split24((double)r.w[h * r.w_stride], mw, ew, nw);
    if (mw == 0) continue;
    for (int i = 0; i < 20; ++i)
      if (acc.l[i]) tot.add((uint64_t)acc.l[i] * (uint64_t)mw, ew + kDotBase + 32 * i + 544, nw);
  }
  return wide_to_f32(tot, -544);
}

SP_DEV bool certify(double y, double e, float& key) {
  float lo = (float)(y - e), hi = (float)(y + e);
  key = lo + 0.0f;
  return lo == hi;
}

// key of candidate j: float32 nearest to the exact score
SP_DEV float exact_key(const IndexerRow& r, int64_t j) {
  const double g52 = 2.220446049250313e-16;  // 2^-52
  int64_t koff = j * r.k_stride;
  if (!r.relu) {
    double y = 0.0, A = 0.0;
    bool x = true;
    for (int c = 0; c < r.d; ++c) {
      double t = load_f64(r.q, r.qt, c) * load_f64(r.k, r.kt, koff + c);   // exact product
      xadd(y, x, t);
      A += fabs(t);
    }
    if (x) return key_of_exact(y);
    float key;
    if (certify(y, 2.0 * (r.d + 4) * g52 * A + 1e-300, key)) return key;
    return exact_key_slow(r, j);
  }
  double s = 0.0, Es = 0.0, Ar = 0.0, sx = 0.0;
  bool ok = true, xall = true;
  for (int h = 0; h < r.H; ++h) {
    double y = 0.0, A = 0.0;
    bool x = true;
    for (int c = 0; c < r.d; ++c) {
      double t = load_f64(r.q, r.qt, h * r.qh_stride + c) * load_f64(r.k, r.kt, koff + c);
      xadd(y, x, t);
      A += fabs(t);
    }
    double E = 2.0 * (r.d + 4) * g52 * A + 1e-300;
    double w = (double)r.w[h * r.w_stride];
    if (!x) xall = false;
    else if (y > 0.0 && w != 0.0) xadd_prod(sx, xall, w, y);
    if (y > E) {
      s += w * y;
      Es += fabs(w) * E;
      Ar += fabs(w * y);
    } else if (!(y < -E) && w != 0.0) {
      ok = false;
    }
  }
  if (xall) return key_of_exact(sx);
  float key;
  if (ok && certify(s, Es + 2.0 * (r.H + 4) * g52 * Ar + 1e-300, key)) return key;
  return exact_key_slow(r, j);
}

// The same key computed by a group of W aligned lanes (a wave, or a quarter-
// wave so that several candidates are scored at once) for one candidate j
// (group-uniform): lane l takes a contiguous run of 64 / W dimensions of
// every 64 (one vector load of the key row; zeros past d add nothing), heads
// go HB at a time with all their operands loaded before the reduction, and
// the per-head sums are reduced across the group. QL: the row's queries and
// weights are in LDS (qs [H][d], wsg [H], exact float copies); otherwise they
// are read from the inputs. The code is straight-line apart from uniform
// branches on H and on the score mode.
template <int W, bool QL, int HB, bool SLOW>
SP_DEV float group_exact_key_impl(const IndexerRow& r, int64_t j, const float* qs, const float* wsg) {
  const double g52 = 2.220446049250313e-16;
  constexpr int NK = 64 / W;
  const int lane = threadIdx.x & (W - 1);
  const int base = (threadIdx.x & 63) & ~(W - 1);
  const int64_t koff = j * r.k_stride;
  double s = 0.0, Es = 0.0, Ar = 0.0, sx = 0.0;
  bool ok = true, xall = true;
  for (int h0 = 0; h0 < r.H; h0 += HB) {
    double y[HB], A[HB], wv[HB];              // wv: loaded with the operands, used after the reduction
    bool x[HB];
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      y[u] = A[u] = wv[u] = 0.0;
      x[u] = true;
    }
#pragma unroll
    for (int u = 0; u < HB; ++u)
      if (r.relu && h0 + u < r.H) wv[u] = QL ? (double)wsg[h0 + u] : (double)r.w[(h0 + u) * r.w_stride];
    for (int c0 = 0; c0 < r.d; c0 += 64) {
      const int cb = c0 + NK * lane;
      double kv[NK];
      load_run_f64<NK>(r.k, r.kt, koff + cb, r.d - cb, kv);
#pragma unroll
      for (int u = 0; u < HB; ++u) {
        if (h0 + u < r.H) {
          double qv[NK];
          if constexpr (QL) {
#pragma unroll
            for (int i = 0; i < NK; ++i) qv[i] = cb + i < r.d ? (double)qs[(h0 + u) * r.d + cb + i] : 0.0;
          } else {
            load_run_f64<NK>(r.q, r.qt, (h0 + u) * r.qh_stride + cb, r.d - cb, qv);
          }
#pragma unroll
          for (int i = 0; i < NK; ++i) {
            const double t = qv[i] * kv[i];   // exact product
            xadd(y[u], x[u], t);
            A[u] += fabs(t);
          }
        }
      }
    }
    if constexpr (W == 16) {
      row16_xreduce<HB>(y, x, A);
    } else {
#pragma unroll
      for (int u = 0; u < HB; ++u) group_xreduce<W>(y[u], x[u], A[u]);
    }
    if (!r.relu) {                             // plain dot: one head
      if (x[0]) return key_of_exact(y[0]);
      float key;
      if (certify(y[0], 2.0 * (r.d + 70) * g52 * A[0] + 1e-300, key)) return key;
      ok = false;
      break;
    }
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      if (h0 + u < r.H) {
        const double E = 2.0 * (r.d + 70) * g52 * A[u] + 1e-300;   // r.d / W + log2 W terms per path
        const double w = wv[u];
        if (!x[u]) xall = false;
        else if (y[u] > 0.0 && w != 0.0) xadd_prod(sx, xall, w, y[u]);
        if (y[u] > E) {
          s += w * y[u];
          Es += fabs(w) * E;
          Ar += fabs(w * y[u]);
        } else if (!(y[u] < -E) && w != 0.0) {
          ok = false;
        }
      }
    }
  }
  if (r.relu && xall) return key_of_exact(sx);
  float key = 0.f;
  if (r.relu && ok && certify(s, Es + 2.0 * (r.H + 4) * g52 * Ar + 1e-300, key)) return key;
  if constexpr (!SLOW) return __builtin_nanf("");   // the caller redoes the row
  float slow = 0.f;
  if (lane == 0) slow = exact_key_slow(r, j);
  return __shfl(slow, base, 64);
}

// qs/wsg (optional, together): the row's queries [H][d] and weights [H]
// already in LDS as float (exact copies of the bf16/f32 inputs). HB heads
// are tracked at once (fewer registers with a smaller batch, more latency).
// SLOW = false: a key that neither the exact path nor the bound settles is
// returned as NaN instead of being formed in the wide accumulator (kept out
// of register-tight kernels; the caller then redoes the row elsewhere).
template <int W, int HB = 4, bool SLOW = true>
SP_DEV float group_exact_key(const IndexerRow& r, int64_t j, const float* qs = nullptr, const float* wsg = nullptr) {
  return qs ? group_exact_key_impl<W, true, HB, SLOW>(r, j, qs, wsg)
            : group_exact_key_impl<W, false, HB, SLOW>(r, j, nullptr, nullptr);
}
SP_DEV float wave_exact_key(const IndexerRow& r, int64_t j) { return group_exact_key<64>(r, j); }

// Rigorous bound on |score~ - key| for a row scored by the indexer kernels
// from its inputs: CO = sum over the group's heads and dims of |w_h q_hc|
// (summed in float32 in any order), KM = max |k| over the row's keys.
SP_DEV float eps_of(const IndexerParams& x, float CO, float KM) {
  const double u = 1.0 / 8388608.0;
  auto gam = [&](double n) { return n * u / (1.0 - n * u); };
  const double C = 1.25 * (gam(x.d_I + 2) + gam(x.hpg + 2) * (1.0 + gam(x.d_I + 2)) + u);
  // CO was summed in float32: inflate by its own rounding bound
  const double e = C * (double)CO * (1.0 + gam(x.hpg * x.d_I + 2)) * (double)KM * (1.0 + 1e-6) + 1e-30;
  return (float)e * (1.0f + 1e-6f);
}

// The same bound for one row by a whole workgroup: KM from the indexer's
// per-chunk maxima x.kmax[(b * G_k + kg) * nchunk + c] over the chunks that
// hold keys 0..L-1, CO from the row's query and weights. Every thread calls
// it; red holds >= 32 floats; two barriers.
SP_DEV float row_eps(const IndexerParams& x, const IndexerRow& ir, int b, int kg, int L, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nch = min(x.nchunk, (L + x.chunk - 1) / x.chunk);
  const float* km_row = x.kmax + ((int64_t)b * x.G_k + kg) * x.nchunk;
  float km = 0.f;
  for (int i = tid; i < nch; i += blockDim.x) km = fmaxf(km, km_row[i]);
  float coef = 0.f;
  for (int e = tid; e < ir.H * ir.d; e += blockDim.x) {
    const int h = e / ir.d, cc = e % ir.d;
    const float qv = fabsf((float)load_f64(ir.q, ir.qt, h * ir.qh_stride + cc));
    const float wv = ir.relu ? fabsf(ir.w[h * ir.w_stride]) : 1.f;
    coef = fmaf(wv, qv, coef);
  }
  km = wave_max(km);
  coef = wave_sum(coef);
  if (lane == 0) {
    red[wid] = km;
    red[16 + wid] = coef;
  }
  __syncthreads();
  float KM = 0.f, CO = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    KM = fmaxf(KM, red[w]);
    CO += red[16 + w];
  }
  __syncthreads();
  return eps_of(x, CO, KM);
}

// Block key: float32 nearest to (1/bs) * sum_{t<bs} q . k[t]; bs a power of two.
SP_DEV float exact_block_key(const void* q, int qt, const void* k, int kt, int64_t k_stride,
                             int bs, int log2bs, int d) {
  const double g52 = 2.220446049250313e-16;
  double y = 0.0, A = 0.0;
  bool x = true;
  for (int t = 0; t < bs; ++t)
    for (int c = 0; c < d; ++c) {
      double v = load_f64(q, qt, c) * load_f64(k, kt, t * k_stride + c);   // exact product
      xadd(y, x, v);
      A += fabs(v);
    }
  if (x) return key_of_exact(ldexp(y, -log2bs));
  double e = 2.0 * (bs * d + 8) * g52 * A + 1e-300;
  float key;
  if (certify(ldexp(y, -log2bs), ldexp(e, -log2bs), key)) return key;
  DotAcc acc;
  acc.clear();
  for (int t = 0; t < bs; ++t) exact_dot_acc(acc, q, qt, 0, k, kt, t * k_stride, d);
  return wide_to_f32(acc, kDotBase - log2bs);
}

}  // namespace sp
