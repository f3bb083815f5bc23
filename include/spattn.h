/*
 * libspattn — selective sparse attention on AMD Instinct MI355X (gfx950).
 *
 * A lightweight indexer scores every past key for each query, a per-query
 * top-K picks the visible key set S(i), and attention softmax(q k^T/sqrt(d)) V
 * is computed over S(i) only. Fixed visible sets (sliding window + global
 * tokens, block-sparse selection) are special cases of the same attention call.
 *
 * Sources of the method (the pages this library restates):
 *  - "A Guide to Sparse Attention in Large Models", section 2 (attention
 *    restricted to a visible key set S(i) through a mask) and section 4
 *    (index-based and fused implementations);
 *  - "Sparse Attention for Long-Context LLM Inference", sections on the
 *    lightweight indexer ("coarse filter first, precise compute later") and
 *    on Top-K candidate control;
 *  - "Sparse Attention in 2026: Why It Finally Had to Be Native", DSA
 *    paragraph (a few-head low-precision indexer, top-k key/value entries);
 *  - "Sparse Attention Is Reshaping Production AI", fixed patterns and
 *    learned block routing (mean-pooled block keys, top-k blocks);
 *  - "Sparse Attention" (completesystemdesign.dev), sliding window + global
 *    tokens and block-sparse patterns;
 *  - "Sparse Attention in 2026", DSA list (page-granular selection: the
 *    indexer rates every KV page, attention reads the best pages plus the
 *    mandatory recent pages).
 *
 * Conventions shared by every call
 *  - All tensors are caller-owned device buffers described by spattn_tensor
 *    (strides in elements; the innermost dimension must have stride 1 and
 *    rows must be 16-byte aligned where noted). The library never allocates
 *    device memory, never synchronizes, and keeps no state between calls: a
 *    call validates its arguments on the host and enqueues kernels on
 *    `stream` (a hipStream_t; NULL = the default stream).
 *  - Queries are the last Nq positions of each request's context: the query
 *    in row r of request b sits at position p = ctx_len[b] - Nq + r and sees
 *    keys 0..p (causal). Prefill has Nq = ctx_len, decode has Nq = 1.
 *    `ctx_len` is a device int32 array [B] or NULL (every request holds the
 *    full capacity `ctx` of the key tensors). Values must lie in [Nq, ctx];
 *    they are read on the device and not checked by the host.
 *  - Status codes: every call returns SPATTN_OK or an error; validation ends
 *    before any launch, so a failed call enqueues nothing. Errors raised by
 *    kernels at run time surface at the caller's next stream synchronization.
 *    spattn_last_error_message() returns a thread-local description.
 *  - Workspace: `ws` is caller-owned device scratch of at least the size the
 *    matching *_workspace() query returns for the same arguments (0 is
 *    allowed where the query returns 0). It need not be initialized.
 */
#ifndef SPATTN_H
#define SPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPATTN_API __attribute__((visibility("default")))

enum spattn_status {
  SPATTN_OK = 0,
  SPATTN_ERR_INVALID_ARG = 1,   /* null pointer, bad shape or stride, bad parameter */
  SPATTN_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype, head dim, sizes) */
  SPATTN_ERR_WORKSPACE = 3,     /* ws_bytes below the size the *_workspace() query gives */
  SPATTN_ERR_NO_DEVICE = 4,     /* no usable gfx950 device */
  SPATTN_ERR_LAUNCH = 5         /* the HIP runtime refused a launch */
};

enum spattn_dtype { SPATTN_F32 = 0, SPATTN_BF16 = 1, SPATTN_FP8_E4M3 = 2, SPATTN_I32 = 3 };

/* A strided view of a device buffer. ndim <= 4; unused trailing entries ignored. */
typedef struct spattn_tensor {
  void* data;
  int32_t dtype;       /* enum spattn_dtype; FP8_E4M3 is OCP E4M3FN (bias 7, max 448, no inf) */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];   /* in elements; 0 broadcasts */
} spattn_tensor;

/* Indexer score s(i,j) of key j for selection group g of query row i. */
enum spattn_score_mode {
  /* s = q_I[i,g] . k_I[j]  (one indexer head per group) */
  SPATTN_SCORE_DOT = 0,
  /* s = sum over the group's heads h of w[i,h] * max(0, q_I[i,h] . k_I[j]) */
  SPATTN_SCORE_WEIGHTED_RELU = 1
};

/* Indexer inputs ("Sparse Attention for Long-Context LLM Inference",
 * lightweight indexer; "Sparse Attention in 2026", DSA lightning indexer).
 * The indexer takes no positions: its scores depend on content only. */
typedef struct spattn_indexer {
  spattn_tensor q_idx;    /* [B, Nq, H_I, d_I]  f32 | bf16 */
  spattn_tensor k_idx;    /* [B, ctx, G_k, d_I] f32 | bf16 | fp8; G_k = 1 (shared by all
                             selection groups) or G_k = G_sel (one key head per group) */
  spattn_tensor w;        /* [B, Nq, H_I] f32 head weights, strides may be 0 (broadcast);
                             ignored (may be empty) in DOT mode */
  int32_t score_mode;     /* enum spattn_score_mode */
  int32_t heads_per_group;/* H_I / G_sel; must be 1 in DOT mode */
} spattn_indexer;

/* How the visible key set S(i) of each query row is formed. */
enum spattn_sel_mode {
  SPATTN_SEL_DENSE = 0,          /* S = all keys 0..p (the conservative fallback) */
  SPATTN_SEL_INDEX = 1,          /* S = explicit index list (e.g. from spattn_topk) */
  SPATTN_SEL_WINDOW_GLOBAL = 2,  /* S = {p-window+1..p} U {0..n_global-1} U {multiples of
                                    stride}, within 0..p */
  SPATTN_SEL_BLOCKS = 3,         /* S = selected blocks U {p-window+1..p}, within 0..p */
  SPATTN_SEL_PAGES = 4           /* S = every token of the listed pages, within 0..p */
};

typedef struct spattn_selection {
  int32_t mode;          /* enum spattn_sel_mode */
  spattn_tensor idx;     /* INDEX: int32 [B, G_sel, Nq, K], ascending key positions, -1
                            padded; G_sel divides H_q and G_sel | H_kv or H_kv | G_sel.
                            BLOCKS: int32 [B, G_sel, Nq, nb] block ids, -1 padded;
                            G_sel divides H_q and query head h reads list
                            h / (H_q / G_sel) (G_sel = H_q: one list per head).
                            PAGES: int32 [B, G_sel, Nq, np] page ids (page pg = tokens
                            pg*block_size .. pg*block_size+block_size-1), ascending, -1
                            padded (e.g. from spattn_page_select); G_sel as for INDEX. */
  int32_t window;        /* keys in the sliding window, the query itself included */
  int32_t n_global;      /* WINDOW_GLOBAL: tokens 0..n_global-1 are visible to all rows */
  int32_t block_size;    /* BLOCKS: tokens per block; PAGES: tokens per page (power of two) */
  int32_t stride;        /* WINDOW_GLOBAL: when > 0 every token at a multiple of stride is
                            visible too (local window plus dilated stride, "Sparse Attention
                            Is Reshaping Production AI", Fixed Patterns); 0 = none */
} spattn_selection;

/* Paged K/V storage: the keys and values of all requests live in a pool of
 * fixed-size pages, and a page table maps each request's logical pages to pool
 * pages. Logical token j of request b is row j mod page_size of pool page
 * page_table[b, j / page_size]. */
typedef struct spattn_kv_pages {
  spattn_tensor page_table;   /* int32 [B, max_pages]; entries of pages that hold tokens
                                 0..ctx_len[b]-1 must lie in [0, n_pages) (read on the
                                 device, not checked by the host); others are not read */
  int32_t page_size;          /* tokens per page: a power of two in 1..4096 */
} spattn_kv_pages;

/* ------------------------------------------------------------------------
 * spattn_index_scores — indexer scores for every (query row, past key).
 * Source: "Sparse Attention for Long-Context LLM Inference" (lightweight
 * indexer outputs candidate scores for historical positions); "Sparse
 * Attention in 2026" (DSA: few-head low-precision indexer, ReLU-gated heads).
 *
 *  scores_out: f32 [B, G_sel, Nq, ctx]; entry (b,g,r,j) for j <= p is the
 *              score computed in float32 (MFMA or FMA accumulation); entries
 *              with j > p are unspecified.
 *  err_out:    optional f32 [B, G_sel, Nq]: a rigorous bound on
 *              |scores_out - key| over the row, where key is the float32
 *              nearest to the exact score. spattn_topk uses it to return
 *              oracle-exact index sets.
 *  Limits: d_I <= 256; f32 q_idx requires f32 k_idx.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_index_scores_workspace(const spattn_indexer* ix);
SPATTN_API int spattn_index_scores(const spattn_indexer* ix, const int32_t* ctx_len,
                                   const spattn_tensor* scores_out, float* err_out,
                                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_topk — per-row top-K of past keys.
 * Source: "Sparse Attention for Long-Context LLM Inference", Top-K section
 * (cap on candidates per step); "Sparse Attention in 2026", DSA paragraph
 * (top-k key/value entries per query).
 *
 * Row (b,g,r) has candidates 0..p. The selected set is the min(K, p+1)
 * candidates largest by (score descending, index ascending); written to
 * idx_out int32 [B, G, Nq, K] in ascending index order, -1 padded, with the
 * count in count_out int32 [B, G, Nq] (optional).
 *
 *  flags = 0: selection on the float32 values in `scores` as given.
 *  flags = SPATTN_TOPK_CERTIFIED: `scores`/`err` come from spattn_index_scores
 *      on indexer `ix`; selection is made on the exact keys (float32 nearest
 *      to the exact score), with near-ties rescored exactly, so the result
 *      equals exhaustive selection on exact keys.
 *  flags = SPATTN_TOPK_FUSED_INDEX: `scores` and `err` are NULL; the scores are
 *      computed from `ix` inside (no score matrix is materialized) and the
 *      selection is certified as above.
 *  Limits: 1 <= K <= 16384.
 * ---------------------------------------------------------------------- */
#define SPATTN_TOPK_CERTIFIED 1u
#define SPATTN_TOPK_FUSED_INDEX 2u
SPATTN_API size_t spattn_topk_workspace(const spattn_tensor* scores, const spattn_indexer* ix,
                                        int32_t k, uint32_t flags);
SPATTN_API int spattn_topk(const spattn_tensor* scores, const float* err,
                           const spattn_indexer* ix, const int32_t* ctx_len, int32_t k,
                           uint32_t flags, const spattn_tensor* idx_out, int32_t* count_out,
                           void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_page_select — page-granular selection.
 * Source: "Sparse Attention in 2026: Why It Finally Had to Be Native", DSA
 * list (the indexer rates every KV page; attention reads the top-rated
 * pages plus the mandatory recent/local pages, whole, without compression).
 *
 * Row (b,g,r) at position p: page pg covers tokens pg*P .. pg*P+P-1. The
 * n_local most recent pages (the one holding p and those before it) are
 * always read. Every earlier page is a candidate keyed by the largest
 * selection key among its tokens within 0..p (the page does not say how
 * token ratings combine; this is the reading the library takes), and the
 * min(top_pages, #candidates) best by (key descending, page ascending) are
 * added. pg_idx_out int32 [B, G, Nq, top_pages + n_local] receives the page
 * ids ascending, -1 padded; pg_count_out int32 [B, G, Nq] (optional) the
 * number of pages.
 *
 *  scores: f32 [B, G, Nq, ctx] token scores (entries past p are not read).
 *  flags = 0: keys are the float32 scores as given.
 *  flags = SPATTN_TOPK_CERTIFIED: scores and err come from
 *      spattn_index_scores on indexer ix; keys are the exact token keys (the
 *      float32 nearest to the exact score), near-ties rescored exactly, so
 *      the page list equals exhaustive selection on exact keys.
 *  flags = SPATTN_TOPK_FUSED_INDEX: scores and err are NULL; the call scores
 *      the tokens from ix itself (into the workspace, with the page keys
 *      taken in the indexer's epilogue where its MFMA kernel applies and P is
 *      32..512) and selects as with SPATTN_TOPK_CERTIFIED.
 *  Limits: P a power of two in 1..4096; ceil(ctx / P) <= 16384;
 *  top_pages, n_local >= 0 with top_pages + n_local >= 1; top_pages <= 16384.
 *  Workspace (the query takes the same scores or indexer and flags): fused,
 *  the scores [B, G, Nq, ctx] f32 and the indexer's per-chunk maxima of |k|,
 *  plus the page keys;
 *  otherwise the page keys of every row when there are at most 512 rows
 *  (B * G * Nq), rows * ceil(ctx / P) * 4 bytes, else nothing.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_page_select_workspace(const spattn_tensor* scores, const spattn_indexer* ix,
                                               int32_t page_size, int32_t top_pages, int32_t n_local,
                                               uint32_t flags);
SPATTN_API int spattn_page_select(const spattn_tensor* scores, const float* err,
                                  const spattn_indexer* ix, const int32_t* ctx_len,
                                  int32_t page_size, int32_t top_pages, int32_t n_local,
                                  uint32_t flags, const spattn_tensor* pg_idx_out,
                                  int32_t* pg_count_out, void* ws, size_t ws_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Two-level selection.
 * Source: "Sparse Attention Is Reshaping Production AI", per-token routing
 * (a coarse block pass identifies candidate regions cheaply, a fine pass
 * picks the top-K tokens from within them; together they beat either alone).
 *
 * spattn_pool_index_keys: k_blocks_out f32 [B, ctx / block_size, G_k, d_I]
 *   receives, for every complete block of each request, the mean of its
 *   tokens' indexer keys (summed in float64, rounded once to float32). A
 *   decode loop keeps this cache and extends it one block at a time.
 * spattn_topk_two_level: row (b,g,r) at position p scores its complete past
 *   blocks {beta : block_size*beta + block_size - 1 <= p} with the indexer's
 *   own score (ix's queries and weights on k_blocks) and keeps the
 *   min(top_blocks, #blocks) best by (key desc, block asc); the candidates are
 *   their tokens plus the tokens of p's own incomplete block; the min(k,
 *   #candidates) best candidates by (token key desc, position asc) are written
 *   ascending to idx_out int32 [B, G, Nq, k], -1 padded (counts optional).
 *   Keys are exact as for SPATTN_TOPK_CERTIFIED (float32 nearest to the exact
 *   score; near-ties rescored exactly), so the result equals exhaustive
 *   two-level selection on exact keys.
 *  Limits: block_size a power of two; ctx / block_size <= 8192;
 *  (top_blocks + 1) * block_size <= 8192; k <= 16384. No workspace.
 * ---------------------------------------------------------------------- */
SPATTN_API int spattn_pool_index_keys(const spattn_indexer* ix, const int32_t* ctx_len, int32_t block_size,
                                      const spattn_tensor* k_blocks_out, void* stream);
SPATTN_API size_t spattn_topk_two_level_workspace(const spattn_indexer* ix, const spattn_tensor* k_blocks,
                                                  int32_t block_size, int32_t top_blocks, int32_t k);
SPATTN_API int spattn_topk_two_level(const spattn_indexer* ix, const spattn_tensor* k_blocks,
                                     const int32_t* ctx_len, int32_t block_size, int32_t top_blocks,
                                     int32_t k, const spattn_tensor* idx_out, int32_t* count_out,
                                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_index_block_select — blockwise selection per GQA group.
 * Source: "Sparse Attention in 2026: Why It Finally Had to Be Native", MSA
 * paragraph (an index branch scores and picks the top-k KV blocks for each
 * GQA group; the main branch attends exactly over them).
 *
 * Row (b,g,r) at position p: the coarse pass of spattn_topk_two_level alone.
 * Every complete past block {beta : block_size*beta + block_size - 1 <= p}
 * is keyed by the indexer's own score on its mean indexer key in k_blocks
 * (from spattn_pool_index_keys), exact as for SPATTN_TOPK_CERTIFIED, and the
 * min(top_blocks, #blocks) best by (key desc, block asc) are written
 * ascending to blk_idx_out int32 [B, G, Nq, top_blocks], -1 padded; counts
 * optional. G is the indexer's selection-group count: with one group per KV
 * head the list serves every query head of that group, as a BLOCKS selection
 * of spattn_sparse_attn_fwd (block lists [B, G, Nq, nb]).
 *  Limits: block_size a power of two; ctx / block_size <= 8192;
 *  top_blocks <= 16384. No workspace.
 * ---------------------------------------------------------------------- */
SPATTN_API int spattn_index_block_select(const spattn_indexer* ix, const spattn_tensor* k_blocks,
                                         const int32_t* ctx_len, int32_t block_size, int32_t top_blocks,
                                         const spattn_tensor* blk_idx_out, int32_t* blk_count_out, void* stream);

/* ------------------------------------------------------------------------
 * spattn_block_select — block routing for block-sparse attention.
 * Source: "Sparse Attention Is Reshaping Production AI", Learned Block
 * Routing (keys mean-pooled per block, unscaled dot product with the query,
 * top-k blocks); "Sparse Attention" (completesystemdesign.dev), NSA/MoBA-style
 * block selection.
 *
 * For query row (b,h,r) at position p the eligible blocks are the complete
 * past blocks {beta : block_size*beta + block_size - 1 <= p}. Each is scored by
 * the float32 nearest to the exact mean over its keys of q.k (head h's own q
 * and its KV head's k), and the min(top_blocks, #eligible) best by
 * (score descending, block ascending) are written ascending to
 * blk_idx_out int32 [B, H_q, Nq, top_blocks], -1 padded; counts optional.
 *  q: [B, H_q, Nq, d] bf16|f32; k: [B, H_kv, ctx, d] same dtype; d in {64,128}.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_block_select_workspace(const spattn_tensor* q, const spattn_tensor* k,
                                                int32_t block_size, int32_t top_blocks);
SPATTN_API int spattn_block_select(const spattn_tensor* q, const spattn_tensor* k,
                                   const int32_t* ctx_len, int32_t block_size,
                                   int32_t top_blocks, const spattn_tensor* blk_idx_out,
                                   int32_t* blk_count_out, void* ws, size_t ws_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------
 * spattn_sparse_attn_fwd — attention restricted to S(i).
 * Source: "A Guide to Sparse Attention in Large Models", section 2 (softmax
 * over the visible key set, everything else masked) and sections 4.2-4.3
 * (index-based and fused implementations that touch only the selected keys).
 *
 *  q: [B, H_q, Nq, d], k, v: [B, H_kv, ctx, d], same dtype (bf16 or f32),
 *     d in {64, 128}, H_kv divides H_q (GQA/MQA). Rows 16-byte aligned.
 *  scale: logit scale; 0 means 1/sqrt(d).
 *  o_out: f32 [B, H_q, Nq, d]; lse_out: optional f32 [B, H_q, Nq], natural
 *     log of the softmax denominator including the scale. A row with an empty
 *     visible set gets O = 0 and LSE = -inf.
 * Index entries outside 0..p and -1 padding are ignored.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_sparse_attn_fwd_workspace(const spattn_tensor* q, const spattn_tensor* k,
                                                   const spattn_selection* sel);
SPATTN_API int spattn_sparse_attn_fwd(const spattn_tensor* q, const spattn_tensor* k,
                                      const spattn_tensor* v, const int32_t* ctx_len,
                                      float scale, const spattn_selection* sel,
                                      const spattn_tensor* o_out, float* lse_out, void* ws,
                                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_sparse_attn_fwd_noalloc — spattn_sparse_attn_fwd for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. It takes no workspace:
 * the kernels' scratch (the decode gather's split partials) lives in a fixed
 * per-device array of spattn_noalloc_scratch_bytes() bytes (32 MiB) that
 * the library holds on every device it runs on until the process ends.
 *
 * Arguments, layouts and results are those of spattn_sparse_attn_fwd (the
 * same kernels run). A call whose workspace query exceeds the array's size
 * returns SPATTN_ERR_WORKSPACE before touching the device (routed blocks at
 * prefill sizes do; decode index lists do not). Nothing is allocated and
 * nothing is synchronized. All calls on one device share the array: calls
 * ordered on one stream are safe, calls that overlap in time on one device
 * (other streams or host threads) race on it.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_noalloc_scratch_bytes(void);
SPATTN_API int spattn_sparse_attn_fwd_noalloc(const spattn_tensor* q, const spattn_tensor* k,
                                              const spattn_tensor* v, const int32_t* ctx_len,
                                              float scale, const spattn_selection* sel,
                                              const spattn_tensor* o_out, float* lse_out, void* stream);

/* ------------------------------------------------------------------------
 * spattn_sparse_attn_fwd_paged — the same attention over paged K/V storage
 * (the serving layout in which the pages of "Sparse Attention in 2026", DSA
 * list, are the unit of selection and of reading).
 *
 *  k_pool, v_pool: [n_pages, H_kv, page_size, d], same dtype as q (bf16 or
 *     f32), d in {64, 128}, rows 16-byte aligned; n_pages * page_size < 2^31.
 *  pages: the page table and page size; the logical capacity is
 *     ctx = max_pages * page_size and ctx_len values must lie in [Nq, ctx].
 *  Every selection mode is accepted; INDEX and PAGES lists with bf16, d = 128
 *  take the gather kernel, the others a generic kernel. Everything else as
 *  spattn_sparse_attn_fwd.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_sparse_attn_fwd_paged_workspace(const spattn_tensor* q,
                                                         const spattn_tensor* k_pool,
                                                         const spattn_kv_pages* pages,
                                                         const spattn_selection* sel);
SPATTN_API int spattn_sparse_attn_fwd_paged(const spattn_tensor* q, const spattn_tensor* k_pool,
                                            const spattn_tensor* v_pool,
                                            const spattn_kv_pages* pages,
                                            const int32_t* ctx_len, float scale,
                                            const spattn_selection* sel,
                                            const spattn_tensor* o_out, float* lse_out,
                                            void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_sparse_attn_bwd — gradients of the sparse attention over the same
 * visible sets. Source: "Sparse Attention in 2026: Why It Finally Had to Be
 * Native" (natively trainable sparsity: forward and backward run over the
 * selected set; the speedup covers training, not only serving).
 *
 * For the forward O = spattn_sparse_attn_fwd(q, k, v, sel) and an upstream
 * gradient d_o, writes dq = d(sum d_o*O)/dq, dk, dv (GQA: a KV head gathers
 * the gradients of all its query heads): with P the softmax over S(i),
 * dV = P^T dO, dS = P (dO V^T - rowsum(dO * O)), dq = scale dS K,
 * dK = scale dS^T Q.
 *  q, k, v, ctx_len, scale, sel: as passed to the forward (contiguous K/V,
 *     every selection mode); o f32 [B, H_q, Nq, d] and lse f32 [B, H_q, Nq]:
 *     the forward's outputs; d_o, dq_out f32 [B, H_q, Nq, d];
 *     dk_out, dv_out f32 [B, H_kv, ctx, d] (overwritten).
 *  ws, ws_bytes: device workspace of at least
 *     spattn_sparse_attn_bwd_workspace(q, k, sel) bytes (caller-owned, no
 *     initial contents needed; null with 0 when that is 0). The window
 *     pattern (WINDOW_GLOBAL without stride, bf16, d = 128) needs one slot
 *     of 64 keys x 128 dims x 2 floats per (request, query head, key tile,
 *     band position): each query tile writes its share of a band key tile's
 *     dK/dV to its slot and a second kernel sums them; every other case
 *     needs none. SPATTN_ERR_WORKSPACE if it is too small (nothing launched).
 *  float32 arithmetic; the other shares of dk/dv are accumulated with float
 *  atomics, so their low bits depend on the order in which rows finish.
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_sparse_attn_bwd_workspace(const spattn_tensor* q, const spattn_tensor* k,
                                                   const spattn_selection* sel);
SPATTN_API int spattn_sparse_attn_bwd(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                                      const int32_t* ctx_len, float scale, const spattn_selection* sel,
                                      const spattn_tensor* o, const float* lse, const spattn_tensor* d_o,
                                      const spattn_tensor* dq_out, const spattn_tensor* dk_out,
                                      const spattn_tensor* dv_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_nsa_fwd — three-branch NSA attention.
 * Source: "Sparse Attention in 2026: Why It Finally Had to Be Native", NSA
 * paragraph (coarse compression of token blocks mean-pooled into single
 * entries, fine-grained selection of the top blocks by the compression
 * branch's own scores, a sliding window, all feeding a learned gate);
 * "Sparse Attention" (completesystemdesign.dev), three parallel paths.
 *
 * For query row (b,h,r) at position p, with each branch's own softmax:
 *  o_cmp: attention over the per-block means of K and V of the complete past
 *         blocks {beta : block_size*beta + block_size - 1 <= p} (the means
 *         are formed here and kept in the cache dtype);
 *  o_sel: attention over the tokens of the blocks listed in blk_idx
 *         int32 [B, H_q, Nq, nb] (e.g. from spattn_block_select, whose scores
 *         q . mean(k) are the compression branch's logits), within 0..p;
 *  o_win: attention over the keys p-window+1..p;
 *  o_out f32 [B, H_q, Nq, d] = g0 o_cmp + g1 o_sel + g2 o_win with
 *  gates f32 [B, H_q, Nq, 3] (the learned gate's outputs, given). A branch
 *  with nothing visible contributes 0.
 *  q, k, v as for spattn_sparse_attn_fwd; block_size a power of two.
 *  Workspace: the pooled K and V, the three branch outputs and the block
 *  attention's scratch (the query gives the size).
 * ---------------------------------------------------------------------- */
SPATTN_API size_t spattn_nsa_fwd_workspace(const spattn_tensor* q, const spattn_tensor* k, int32_t block_size,
                                           const spattn_tensor* blk_idx, int32_t window);
SPATTN_API int spattn_nsa_fwd(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                              const int32_t* ctx_len, float scale, int32_t block_size,
                              const spattn_tensor* blk_idx, int32_t window, const spattn_tensor* gates,
                              const spattn_tensor* o_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spattn_quest_page_bounds / spattn_quest_select — query-aware page selection
 * without a trained indexer.
 * Source: "Sparse Attention" (completesystemdesign.dev), inference-only
 * alternatives (Quest-style page-wise KV selection: the page idea of DSA at
 * serving time, no retraining). The page names no criterion; the library
 * takes Quest's published one (Tang et al., 2024): per page and channel the
 * smallest and largest key of the page's tokens, and for a query the bound
 * sum_c max(q_c min_c, q_c max_c), the largest q . x over the box the keys
 * span, so no token of the page scores above it.
 *
 * spattn_quest_page_bounds: for every complete page pg < ctx_len[b] / P of
 *  every request, bounds_out[b, pg, h, 0:d] = channel-wise minimum and
 *  bounds_out[b, pg, h, d:2d] = maximum of the keys of that page's P tokens
 *  (KV head h). Exact (no rounding). Entries of other pages are not written.
 *  k_pool [n_pages, H_kv, P, d] and pages as for spattn_sparse_attn_fwd_paged;
 *  bounds_out [B, max_pages, H_kv, 2d] in k_pool's dtype, rows 16-byte
 *  aligned. A decode loop refreshes a page's entry once the page is full.
 *
 * spattn_quest_select: row (b, g, r) at position p = ctx_len[b] - Nq + r.
 *  Selection group g of G (H_kv divides G, G divides H_q, H_q / G <= 16)
 *  serves query heads g*H_q/G .. (g+1)*H_q/G - 1. The n_local >= 1 most
 *  recent pages (the one holding p and those before it, so every candidate
 *  page is complete) are always read. Each earlier page is a candidate whose
 *  key is the float32 nearest to the exact sum over the group's heads of
 *  their bounds for that page (bf16/f32 products exact in float64, the sum
 *  certified, an exact wide sum near a rounding boundary), and the
 *  min(top_pages, #candidates) best by (key descending, page ascending)
 *  are added. pg_idx_out int32 [B, G, Nq, top_pages + n_local]: logical page
 *  ids ascending, -1 padded (feed to spattn_sparse_attn_fwd_paged with
 *  SPATTN_SEL_PAGES); pg_count_out int32 [B, G, Nq] (optional).
 *  q [B, H_q, Nq, d] in the bounds' dtype (f32 or bf16), d 64 or 128.
 *  Limits: P a power of two in 1..4096; max_pages <= 16384; top_pages <= 16384.
 *  Workspace: B * G * Nq * max_pages * 4 bytes (the page keys).
 * ---------------------------------------------------------------------- */
SPATTN_API int spattn_quest_page_bounds(const spattn_tensor* k_pool, const spattn_kv_pages* pages,
                                        const int32_t* ctx_len, const spattn_tensor* bounds_out, void* stream);
SPATTN_API size_t spattn_quest_select_workspace(const spattn_tensor* q, const spattn_tensor* bounds,
                                                int32_t page_size, int32_t top_pages, int32_t n_local,
                                                const spattn_tensor* pg_idx_out);
SPATTN_API int spattn_quest_select(const spattn_tensor* q, const spattn_tensor* bounds, const int32_t* ctx_len,
                                   int32_t page_size, int32_t top_pages, int32_t n_local,
                                   const spattn_tensor* pg_idx_out, int32_t* pg_count_out, void* ws,
                                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ helpers */
SPATTN_API const char* spattn_status_string(int status);
SPATTN_API const char* spattn_version(void);
/* Thread-local message describing the last failed call on this thread. */
SPATTN_API const char* spattn_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* SPATTN_H */
