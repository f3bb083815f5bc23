// Page-granular selection ("Sparse Attention in 2026: Why It Finally Had to Be
// Native", DSA list: the indexer rates every KV page, attention reads the
// best pages plus the mandatory recent pages, whole).
//
// Row (b, g, r) at position p: page pg holds tokens pg*P .. pg*P+P-1. The
// n_local pages ending with page p/P are always read; every earlier page is a
// candidate whose key is the largest key among its tokens (within 0..p), and
// the top_pages candidates largest by (key descending, page ascending) join
// them. The list is written ascending.
//
// One 512-thread workgroup per row:
//  1. page keys: the row's scores are read once, coalesced (four tokens per
//     lane when the row is 16-byte aligned), and folded per page by lane
//     shuffles; pages wider than a wave's sweep are merged by LDS atomics.
//     Keys stay in LDS (up to kMaxPages candidates).
//  2. radix select of the top_pages-th largest page key t.
//  3. uncertified: pages above t are in, pages equal to t go in by index.
//     Certified (scores within eps of the exact keys): pages whose computed key
//     is above t + 2 eps are in the exact selection and pages below t - 2 eps
//     are out. A band page's exact key is the largest exact key among its
//     tokens, and only tokens whose computed score reaches the page's computed
//     key - 2 eps can hold it (any other token's exact key lies below the
//     exact key of the page's best computed token). Those tokens are rescored
//     exactly, and the remaining slots go to the band's best by (exact key
//     descending, page ascending).
#include "common.h"
#include "exact.h"
#include "internal.h"
#include "rowselect.h"

namespace sp {

constexpr int kPsThreads = 512;
constexpr int kPsBandCap = 2048;

struct PsSmem {
  uint32_t pk[kMaxPages];        // order keys of the candidate pages
  uint32_t hist[4096];
  uint32_t band_j[kPsBandCap];
  uint32_t band_k[kPsBandCap];
  uint32_t sc[16];
  uint32_t run[4];
};

// Keys of pages 0..npc-1 from the scores of tokens 0..ntok-1 (ntok covers the
// candidate pages, cut at p); pk is zeroed first (0 is below every float key).
template <int T>
SP_DEV void page_keys(const float* s, int ntok, int lgP, int npc, uint32_t* pk) {
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < npc; i += T) pk[i] = 0u;
  __syncthreads();
  const bool vec = lgP >= 2 && (((uintptr_t)s) & 15) == 0;
  const int lg_per = vec ? 2 : 0;                 // log2 tokens per lane
  const int lgG = lgP - lg_per;                   // log2 lanes per page
  const int lim = lgG < 6 ? lgG : 6;              // shuffle steps inside a wave
  const bool whole = lgG <= 6;                    // one lane group holds the whole page
  constexpr int U = 4;
  const int step = T << lg_per;                   // tokens per sweep of the workgroup
  for (int base = 0; base < ntok; base += step * U) {
    uint32_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t0 = base + u * step + (tid << lg_per);
      if (vec) {
        if (t0 + 3 < ntok) {
          const f32x4 v = *(const f32x4*)(s + t0);
          m[u] = max(max(f32_order_key(v[0]), f32_order_key(v[1])), max(f32_order_key(v[2]), f32_order_key(v[3])));
        } else {
          uint32_t mm = 0u;
          for (int e = 0; e < 4; ++e)
            if (t0 + e < ntok) mm = max(mm, f32_order_key(s[t0 + e]));
          m[u] = mm;
        }
      } else {
        m[u] = t0 < ntok ? f32_order_key(s[t0]) : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t0 = base + u * step + (tid << lg_per);
      uint32_t v = m[u];
      for (int o = 0; o < lim; ++o) v = max(v, (uint32_t)__shfl_xor((int)v, 1 << o, 64));
      const int page = t0 >> lgP;
      if ((lane & ((1 << lim) - 1)) == 0 && page < npc) {
        if (whole) pk[page] = v;
        else atomicMax(&pk[page], v);
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPsThreads) void page_select_kernel(PageSelParams q) {
  constexpr int T = kPsThreads;
  __shared__ PsSmem sm;
  const TopkParams& p = q.t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x;
  const int r = row % p.Nq, g = (row / p.Nq) % p.G, b = row / (p.Nq * p.G);
  const int L = min(p.ctx_len ? p.ctx_len[b] : p.ctx, p.ctx);
  const int pos = L - p.Nq + r;
  int32_t* out = p.idx + b * p.is[0] + g * p.is[1] + r * p.is[2];
  int32_t* cnt = p.count ? p.count + ((int64_t)b * p.G + g) * p.Nq + r : nullptr;
  const int W = q.width;
  if (pos < 0) {
    for (int i = tid; i < W; i += T) out[i] = -1;
    if (cnt && tid == 0) *cnt = 0;
    return;
  }
  const int lgP = q.lgP;
  const int last = pos >> lgP;
  const int npc = max(0, last + 1 - q.n_local);    // candidate pages 0..npc-1
  const int K = p.K;
  if (npc <= K) {                                   // every page is read
    for (int i = tid; i < W; i += T) out[i] = i <= last ? i : -1;
    if (cnt && tid == 0) *cnt = last + 1;
    return;
  }
  // from here npc > K, so the n_local recent pages all exist and W = K + n_local
  for (int i = tid; i < q.n_local; i += T) out[K + i] = npc + i;
  if (cnt && tid == 0) *cnt = K + q.n_local;
  if (K == 0) return;

  const float* s = p.scores + b * p.ss[0] + g * p.ss[1] + r * p.ss[2];
  page_keys<T>(s, min(npc << lgP, pos + 1), lgP, npc, sm.pk);

  const uint32_t R = (uint32_t)K;
  uint32_t t, above;
  radix_select<T>(npc, R, [&](int i, uint32_t& k) { k = sm.pk[i]; return true; }, sm.hist, sm.sc, t, above);
  uint32_t klo = t, khi = t;
  float E = 0.f;
  IndexerRow ir{};
  if (p.certified) {
    const float tf = order_key_f32(t);
    E = 2.0f * p.err[((int64_t)b * p.G + g) * p.Nq + r] * 1.0001f + 1e-30f;
    klo = f32_order_key(nextafterf(tf - E, -INFINITY));
    khi = f32_order_key(nextafterf(tf + E, INFINITY));
    ir = indexer_row(p.ix, b, g, r);
  }

  // ordered pass 1: pages above the band, the band cached in page order
  if (tid == 0) { sm.run[0] = 0; sm.run[1] = 0; }
  __syncthreads();
  for (int base = 0; base < npc; base += T) {
    const int i = base + tid;
    const uint32_t k = i < npc ? sm.pk[i] : 0u;
    const bool in = i < npc && k > khi;
    const bool bd = i < npc && k >= klo && k <= khi;
    uint32_t nin, nbd;
    const uint32_t bpos = block_prefix<T>(bd, sm.sc, nbd);
    block_prefix<T>(in, sm.sc, nin);
    const uint32_t bslot = sm.run[1] + bpos;
    if (bd && bslot < (uint32_t)kPsBandCap) {
      sm.band_j[bslot] = (uint32_t)i;
      sm.band_k[bslot] = k;
    }
    __syncthreads();
    if (tid == 0) { sm.run[0] += nin; sm.run[1] += nbd; }
    __syncthreads();
  }
  const uint32_t n_in = sm.run[0], n_band = sm.run[1];
  const uint32_t R2 = R - n_in;                    // >= 1: at most R-1 keys exceed t
  const bool cached = n_band <= (uint32_t)kPsBandCap;
  const int P = 1 << lgP;

  // lowest computed score a token may have and still hold the page's exact key
  auto tok_floor = [&](uint32_t ck) { return nextafterf(order_key_f32(ck) - E, -INFINITY); };
  // exact page key by one thread (the uncached fallback)
  auto exkey_thread = [&](int pg, uint32_t ck) -> uint32_t {
    if (!p.certified) return ck;
    const float lo = tok_floor(ck);
    const int j0 = pg << lgP, j1 = min(j0 + P, pos + 1);
    uint32_t bk = 0u;
    for (int j = j0; j < j1; ++j)
      if (s[j] >= lo) bk = max(bk, f32_order_key(exact_key(ir, j)));
    return bk;
  };

  if (cached && p.certified) {                     // one wave per band page
    for (uint32_t e = tid >> 6; e < n_band; e += T / 64) {
      const int pg = (int)sm.band_j[e];
      const float lo = tok_floor(sm.band_k[e]);
      const int j0 = pg << lgP, j1 = min(j0 + P, pos + 1);
      uint32_t bk = 0u;
      for (int jb = j0; jb < j1; jb += 64) {
        const int j = jb + lane;
        uint64_t m = ballot(j < j1 && s[j] >= lo);
        while (m) {
          const int bit = __builtin_ctzll(m);
          m &= m - 1;
          bk = max(bk, f32_order_key(wave_exact_key(ir, jb + bit)));
        }
      }
      if (lane == 0) sm.band_k[e] = bk;
    }
    __syncthreads();
  }

  uint32_t t2, above2;
  if (cached) {
    radix_select<T>((int)n_band, R2, [&](int i, uint32_t& k) { k = sm.band_k[i]; return true; }, sm.hist, sm.sc,
                    t2, above2);
  } else {
    radix_select<T>(npc, R2,
                    [&](int i, uint32_t& k) {
                      const uint32_t ck = sm.pk[i];
                      if (ck < klo || ck > khi) return false;
                      k = exkey_thread(i, ck);
                      return true;
                    },
                    sm.hist, sm.sc, t2, above2);
  }
  const uint32_t need_eq = R2 - above2;

  // ordered pass 2: the selected candidates in ascending page order
  if (tid == 0) { sm.run[0] = 0; sm.run[1] = 0; sm.run[2] = 0; }
  __syncthreads();
  for (int base = 0; base < npc; base += T) {
    const int i = base + tid;
    bool sel = false, bd = false, eq = false;
    uint32_t ck = 0u;
    if (i < npc) {
      ck = sm.pk[i];
      sel = ck > khi;
      bd = ck >= klo && ck <= khi;
    }
    uint32_t nbd;
    const uint32_t brank = sm.run[1] + block_prefix<T>(bd, sm.sc, nbd);
    if (bd) {
      const uint32_t ex = cached ? sm.band_k[brank] : exkey_thread(i, ck);
      eq = ex == t2;
      if (ex > t2) sel = true;
    }
    uint32_t neq;
    const uint32_t erank = sm.run[2] + block_prefix<T>(eq, sm.sc, neq);
    if (eq && erank < need_eq) sel = true;
    uint32_t nsel;
    const uint32_t opos = sm.run[0] + block_prefix<T>(sel, sm.sc, nsel);
    if (sel && opos < R) out[opos] = i;
    __syncthreads();
    if (tid == 0) { sm.run[0] += nsel; sm.run[1] += nbd; sm.run[2] += neq; }
    __syncthreads();
  }
}

hipError_t launch_page_select(const PageSelParams& p, hipStream_t st) {
  const int rows = p.t.B * p.t.G * p.t.Nq;
  hipLaunchKernelGGL(page_select_kernel, dim3(rows), dim3(kPsThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sp
