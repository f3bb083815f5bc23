// Launch parameters shared between the C-ABI layer and the kernel sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sp {

struct View4 {             // a validated strided view (strides in elements)
  const void* p;
  int dt;                  // 0 f32, 1 bf16, 2 fp8, 3 i32
  int64_t n[4];
  int64_t s[4];
};

// ---------------------------------------------------------------- indexer
struct IndexerParams {
  View4 q;                 // [B, Nq, H_I, d_I]
  View4 k;                 // [B, ctx, G_k, d_I]
  const float* w;          // [B, Nq, H_I] f32 (null in DOT mode)
  int64_t ws_[3];
  int B, Nq, H_I, d_I, G_sel, G_k, hpg, relu, ctx;
  const int32_t* ctx_len;
  float* scores;           // [B, G_sel, Nq, ctx]
  int64_t ss[4];
  float* err;              // [B, G_sel, Nq] or null
  float* kmax;             // workspace [B, G_k, nchunk]
  int chunk, nchunk;
  // threshold filter (fused indexer + top-K): keep (key, index) pairs with score >= tau
  const float* tau;        // [B, G_sel, Nq] or null (store every score instead)
  uint32_t* cand;          // [B][nchunk][G_sel * Nq][cap][2]: (order key, key position), 8-byte aligned
  uint32_t* cand_n;        // [B][nchunk][G_sel * Nq] number found (may exceed cap)
  int cap;
  // per-row lists instead (many rows, one selection group): order keys
  // cand[row][cap], positions cand_j[row][cap], counts cand_n[row] (zeroed
  // before the call; a count may exceed cap, the excess is dropped)
  uint32_t* cand_j;
  // page keys (MFMA path only): the largest score of each (selection row, page)
  // as an order key, [B * G_sel * Nq][pk_stride], pages of 1 << pk_lgP keys
  uint32_t* pkeys;
  int64_t pk_stride;
  int pk_lgP;
};
bool index_pagekeys_ok(const IndexerParams& p, int lgP);   // pages of 32..512 keys
int index_chunk(const IndexerParams& p);   // keys per chunk of the chunk maxima (kmax)
bool index_filter_ok(const IndexerParams& p);
bool index_filter_rows_ok(const IndexerParams& p);   // per-row lists (cand_j given)
hipError_t launch_index_filter(const IndexerParams& p, hipStream_t st);   // chunk = 512
size_t indexer_ws_bytes(int B, int G_k, int ctx);
hipError_t launch_index_scores(const IndexerParams& p, hipStream_t st);

// ---------------------------------------------------------------- top-K
struct TopkParams {
  const float* scores;     // [B, G, Nq, ctx]
  int64_t ss[4];
  const float* err;        // [B, G, Nq] or null (then selection on scores as given)
  bool certified;
  IndexerParams ix;        // rescoring inputs when certified
  int B, G, Nq, ctx, K;
  const int32_t* ctx_len;
  int32_t* idx;            // [B, G, Nq, K]
  int64_t is[4];
  int32_t* count;          // [B, G, Nq] or null
  void* ws;                // workspace (few-long-rows schedule)
};
size_t topk_ws_bytes(const TopkParams& p);
hipError_t launch_topk(const TopkParams& p, hipStream_t st);
bool topk_fused_ok(const TopkParams& p);
size_t topk_fused_ws_bytes(const TopkParams& p);
hipError_t launch_topk_fused(const TopkParams& p, hipStream_t st);

// ---------------------------------------------------------------- page select
constexpr int kMaxPages = 16384;   // candidate pages per row held in LDS
struct PageSelParams {
  TopkParams t;            // scores, err, indexer (certified), shapes; t.K = top_pages;
                           // t.idx / t.is: page list [B, G, Nq, width]; t.count
  int lgP, n_local, width; // log2 page size, mandatory recent pages, list width
  void* ws;                // workspace: fused scores and error bounds, staged page keys
  bool fused;              // scores computed here from t.ix (no score matrix given)
};
size_t page_select_ws_bytes(const PageSelParams& p);
hipError_t launch_page_select(const PageSelParams& p, hipStream_t st);
// selection on page keys given as order keys in pkg[row * npmax + page]
// (every candidate page of every row with more candidates than p.t.K),
// taken as they are (p.t.certified false, no scores)
hipError_t launch_page_select_keys(const PageSelParams& p, const uint32_t* pkg, int npmax, hipStream_t st);

// ---------------------------------------------------------------- Quest page selection
struct QuestParams {
  View4 q;                 // [B, Hq, Nq, d]
  View4 kp;                // key pool [n_pages, Hkv, P, d]
  const int32_t* ptab;     // page table [B, maxp]
  int64_t pts[2];
  void* bnd;               // page bounds [B, maxp, Hkv, 2d] in the key dtype: min | max
  int64_t bs[3];
  int B, Hq, Hkv, Nq, d, dt, lgP, maxp, ctx;
  const int32_t* ctx_len;
  PageSelParams sel;       // selection groups, top_pages, n_local, outputs; ws: page keys
};
size_t quest_ws_bytes(const QuestParams& p);
hipError_t launch_quest_bounds(const QuestParams& p, hipStream_t st);
hipError_t launch_quest_select(const QuestParams& p, hipStream_t st);

// ---------------------------------------------------------------- two-level selection
constexpr int kTlMaxCand = 8192;   // blocks per row, and candidate tokens per row
struct TwoLevelParams {
  TopkParams t;            // token indexer (t.ix), shapes, ctx_len, output list [B, G, Nq, K], counts
  float* kp;               // block indexer keys [B, ctx >> lgbs, G_k, d_I] f32
  int64_t kps[4];
  int lgbs, nb;            // log2 block size, blocks kept by the first pick
  bool blocks_only;        // emit the first pick's blocks [B, G, Nq, nb] and stop
};
hipError_t launch_pool_index_keys(const TwoLevelParams& p, hipStream_t st);
hipError_t launch_two_level(const TwoLevelParams& p, hipStream_t st);

// ---------------------------------------------------------------- block select
struct BlockSelectParams {
  View4 q;                 // [B, Hq, Nq, d]
  View4 k;                 // [B, Hkv, ctx, d]
  int B, Hq, Hkv, Nq, ctx, d, bs, log2bs, nb;
  const int32_t* ctx_len;
  int32_t* out;            // [B, Hq, Nq, nb]
  int64_t os[4];
  int32_t* count;
  float* kbar;             // workspace [B, Hkv, ctx/bs, d] f32: per-block key sums
  float* kabs;             // workspace [B, Hkv, ctx/bs] f32: max_c sum_t |k| per block
  double* kbar64;          // workspace [B, Hkv, ctx/bs, d] f64: the same sums in float64
  uint32_t* kexact;        // workspace [B, Hkv, ctx/bs]: 1 when every float64 sum is exact
  uint16_t* kb2;           // workspace [2][B, Hkv, ctx/bs, d] bf16: the float32 sums split in two
                           // (hi + mid within 2^-16 relative), the operands of the MFMA scoring
};
size_t block_select_ws_bytes(int B, int Hkv, int ctx, int d, int bs);
hipError_t launch_block_select(const BlockSelectParams& p, hipStream_t st);

// ---------------------------------------------------------------- attention
struct AttnParams {
  View4 q;                 // [B, Hq, Nq, d]
  View4 k, v;              // [B, Hkv, ctx, d]
  int B, Hq, Hkv, Nq, ctx, d;
  const int32_t* ctx_len;
  float scale;
  int mode;                // 0 dense, 1 index, 2 window/global, 3 blocks, 4 pages,
                           // 5 compressed entries (k, v: per-block means; bs: block size)
  const int32_t* sel;      // index list, block list or page list
  int64_t sels[4];
  int G_sel, K;            // list groups and width (index: keys; blocks: blocks; pages: page
                           // slots times the page size, i.e. one entry per token slot)
  int window, n_global, bs;
  int stride;              // window/global: every stride-th token is visible too (0: none)
  int lgbs;                // pages: log2 of the tokens per listed page
  // paged K/V storage: k, v are pools [n_pages, Hkv, 1 << lgP, d]; logical page
  // pg of request b lives in pool page ptab[b * pts + pg]
  const int32_t* ptab;
  int64_t pts;
  int lgP;
  float* o;                // [B, Hq, Nq, d] f32
  int64_t os[4];
  float* lse;              // [B, Hq, Nq] or null
  void* ws;
  size_t ws_bytes;
  // mode 5 on the tile kernel: each entry is the bf16 pair k + klo (v + vlo),
  // the low parts stored with the strides of k (v); null: one part
  const void* klo;
  const void* vlo;
};
size_t attn_ws_bytes(const AttnParams& p);
// backward over the same visible sets: gradients of sum(dO * O)
struct AttnBwd {
  const float* o;          // forward output [B, Hq, Nq, d]
  int64_t os[4];
  const float* lse;        // forward LSE [B, Hq, Nq]
  const float* dO;         // [B, Hq, Nq, d]
  int64_t dos[4];
  float* dq;               // [B, Hq, Nq, d]
  int64_t dqs[4];
  float* dk;               // [B, Hkv, ctx, d] (zeroed, then accumulated)
  int64_t dks[4];
  float* dv;
  int64_t dvs[4];
  // window pattern on the tile kernel: each query tile's share of a band key
  // tile's dK/dV goes to its own slot here ([B][Hq][ctx tiles][nslot][64 keys
  // x 128 dims x 2], float32) and a reduce kernel sums the slots; null:
  // float atomics instead
  float* part;
  int nslot;
};
hipError_t launch_attention_bwd(const AttnParams& a, const AttnBwd& g, hipStream_t st);
size_t attn_bwd_ws_bytes(const AttnParams& a);
// tiled backward of the dense and window/global patterns (bf16, d = 128)
bool attn_bwd_tile_ok(const AttnParams& a);
hipError_t launch_attn_bwd_tile(const AttnParams& a, const AttnBwd& g, hipStream_t st);
int attn_bwd_slots(const AttnParams& a);   // slots per band key tile (0: no partials for this pattern)
int attn_bwd_zero_rows(const AttnParams& a, const AttnBwd& g);   // dK/dV rows zeroed before the backward
// three-branch NSA attention: compression (mode 5 over the pooled blocks),
// selection (mode 3 without window), window (mode 2), combined by gates
struct NsaParams {
  AttnParams a;            // q, k, v, ctx_len, scale, shapes; sel/sels/K: block lists [B, Hq, Nq, nb]
  const float* gates;      // [B, Hq, Nq, 3] f32: compression, selection, window
  int64_t gs[4];
  float* o;                // [B, Hq, Nq, d] f32
  int64_t os[4];
  void* ws;
};
size_t nsa_ws_bytes(const NsaParams& p);
hipError_t launch_nsa(const NsaParams& p, hipStream_t st);
hipError_t launch_attention(const AttnParams& p, hipStream_t st);
bool attn_tile_ok(const AttnParams& p);
hipError_t launch_attn_tile(const AttnParams& p, hipStream_t st);
bool attn_blocks_ok(const AttnParams& p);
size_t attn_blocks_ws_bytes(const AttnParams& p);
hipError_t launch_attn_blocks(const AttnParams& p, hipStream_t st);

}  // namespace sp
