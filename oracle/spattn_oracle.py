"""CPU oracle for selective sparse attention (test infrastructure only).

This module is the plain, slow, obviously-correct statement of what the GPU
library computes. It is test infrastructure: only the test-suite, the smoke
check and the benchmark's CPU-baseline leg may import it. It shares no code
with the GPU path (the HIP library and its Python binding) and imports nothing
from it; both sides are fed the same seeded inputs.

Everything is computed in float64 from exactly decoded inputs.

What is computed (sources are the five pages on sparse attention):

* Attention restricted to a visible key set S(i): softmax(q k^T / sqrt(d)) V
  with every key outside S(i) masked to -inf before the softmax
  ("A Guide to Sparse Attention in Large Models", section 2 "Core
  Motivation", mask formula, and section 4.1 "Mask-based Implementation").
  The literal "QK^T * Mask + (1-Mask)*(-inf)" formula multiplies 0 by -inf;
  it is read as a masked fill, as the page's own example does.
* Causality: a query at position p sees keys 0..p ("Sparse Attention",
  lower-triangular dense pattern, cost N^2/2).
* Sliding window of w keys including the query itself, plus g global tokens
  at positions 0..g-1 ("Sparse Attention", sliding window + global figure,
  cost N*w + N*g; "A Guide ...", section 2 pattern list), plus, with a stride
  R > 0, every past token at a multiple of R ("Sparse Attention Is Reshaping
  Production AI", Fixed Patterns: local window plus dilated stride).
* Block-sparse selection: keys pooled by mean over 64-token blocks, each
  query scores blocks by an unscaled dot product with the pooled key and keeps
  the top blocks ("Sparse Attention Is Reshaping Production AI", "Learned
  Block Routing" example), restricted here to complete past blocks, unioned
  with the local window.
* Token top-K from a lightweight indexer ("Sparse Attention for Long-Context
  LLM Inference", sections on the lightweight indexer and Top-K;
  "Sparse Attention in 2026", DSA paragraph): score s(i,j) is either
  q_I . k_I,j or sum_h w_h * ReLU(q_I,h . k_I,j), the indexer carries no
  positional encoding, and the K highest scoring past keys are kept.
* Three-branch NSA attention ("Sparse Attention in 2026", NSA paragraph;
  "Sparse Attention" (completesystemdesign.dev), three parallel paths): a
  compression branch attends over the key and value blocks mean-pooled into
  single entries (complete past blocks), a selection branch over the tokens of
  the top blocks chosen by the compression branch's own scores (the pooled-key
  dot products above), and a window branch; each branch has its own softmax
  and a gate weighs them: o = g_cmp o_cmp + g_sel o_sel + g_win o_win. A branch
  with no visible entry contributes 0. The pages fix no precision for the
  compressed entries, so they are the plain block means, exact in float64.
* Two-level selection ("Sparse Attention Is Reshaping Production AI",
  per-token routing: a coarse block pass finds candidate regions, a fine pass
  picks the top-K tokens inside them). Read as: each complete block's indexer
  key is the mean of its tokens' indexer keys, kept in float32 (a per-block
  cache); the coarse pass scores blocks with the indexer's own score on those
  keys and keeps the top_blocks complete past blocks by (key desc, block asc);
  the candidates are the chosen blocks' tokens plus the query's own
  incomplete block, and the fine pass keeps the K best candidates by (token
  key desc, position asc).
* Page-granular selection ("Sparse Attention in 2026: Why It Finally Had to
  Be Native", the DSA list: the indexer rates every 64-token KV page, the
  attention reads the best pages plus the mandatory recent pages, whole).
  The page does not say how token scores become a page rating; it is read
  here as the largest key among the page's visible tokens. The recent pages
  are the n_local pages ending with the one that holds the query position;
  every earlier page competes by (page key descending, page index ascending).
* Blockwise selection per GQA group ("Sparse Attention in 2026", MSA
  paragraph: an index branch scores and picks the top-k KV blocks for each
  GQA group and the main branch attends exactly over them). The page does
  not say how the index branch rates a block; it is read as the indexer's own
  score on the block's mean indexer key (kept in float32, as in the two-level
  coarse pass), over complete past blocks, ranked by (key descending, block
  ascending) with no softmax, and the query's local window is attended too
  (as for the block-sparse pattern), so every row sees at least itself.
* Query-aware page selection without a trained indexer ("Sparse Attention"
  (completesystemdesign.dev), inference-only alternatives: Quest-style
  page-wise KV selection). The page names no criterion; Quest's published one
  (Tang et al., 2024) is taken: each complete page keeps the channel-wise
  minimum m and maximum M of its keys, and a selection group's key for the
  page is the float32 nearest to the exact sum over the group's query heads h
  and channels c of max(q_hc m_c, q_hc M_c) (the largest q . x over the box
  [m, M]). The n_local >= 1 most recent pages are always read and the others
  ranked by (key descending, page ascending).

Selection keys. The pages fix no precision for the scores. Selection is made
on key(j) = the float32 nearest (ties to even) to the exact real-valued score,
with -0 read as +0, ordered by (key descending, index ascending). This key
has one value whatever order a machine sums in, which is what makes index sets
comparable bit for bit. It is obtained by a certified float64 evaluation (the
float32 rounding of every point of a rigorous error interval agrees) and, when
that fails, by exact rational arithmetic.

Pins (tests/test_oracle_pins.py and the fixtures in tests/golden/): index
sets against exact brute force, hand-worked cases and closed forms; masked
attention against torch's scaled-dot-product attention with the same mask;
gradients against torch autograd in float64. The pages print no worked
attention outputs, so the outputs O of the bf16 workloads are parity
unpinned beyond this definition and those identities.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

U52 = 2.0 ** -52

# --------------------------------------------------------------------------
# exact decoding of the storage formats
# --------------------------------------------------------------------------


def _fp8_e4m3fn_value(code: int) -> float:
    """OCP 8-bit E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; 0x7F NaN."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * math.ldexp(m, -9)          # subnormal: m/8 * 2^-6
    return sign * math.ldexp(8 + m, e - 10)      # (1 + m/8) * 2^(e-7)


_FP8_TABLE = np.array([_fp8_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode(a: np.ndarray, fmt: str) -> np.ndarray:
    """Storage array -> float64 (exact)."""
    if fmt == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if fmt == "fp8":
        return _FP8_TABLE[np.asarray(a, dtype=np.uint8)]
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# exact rounding of a rational to float32
# --------------------------------------------------------------------------


def f32_nearest(x: Fraction) -> np.float32:
    """The float32 nearest to the rational x, ties to even (IEEE 754 RNE)."""
    if x == 0:
        return np.float32(0.0)
    neg = x < 0
    a = -x if neg else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if (Fraction(2) ** e) > a:
        e -= 1
    elif (Fraction(2) ** (e + 1)) <= a:
        e += 1
    quantum_exp = max(e, -126) - 23            # spacing of float32 around a
    scaled = a / (Fraction(2) ** quantum_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n * (Fraction(2) ** quantum_exp) > Fraction((2 - 2 ** -23)) * Fraction(2) ** 127:
        val = math.inf
    else:
        val = math.ldexp(n, quantum_exp)
    return np.float32(-val if neg else val)


def _frac(v: float) -> Fraction:
    return Fraction(float(v))


def exact_dot(q: np.ndarray, k: np.ndarray) -> Fraction:
    return sum((_frac(a) * _frac(b) for a, b in zip(q, k)), Fraction(0))


def exact_key_dot(q: np.ndarray, k: np.ndarray) -> np.float32:
    return f32_nearest(exact_dot(q, k))


def exact_key_weighted_relu(qh: np.ndarray, w: np.ndarray, k: np.ndarray) -> np.float32:
    total = Fraction(0)
    for h in range(qh.shape[0]):
        dh = exact_dot(qh[h], k)
        if dh > 0:
            total += _frac(w[h]) * dh
    return f32_nearest(total)


def exact_key_block(q: np.ndarray, kblock: np.ndarray) -> np.float32:
    total = Fraction(0)
    for t in range(kblock.shape[0]):
        total += exact_dot(q, kblock[t])
    return f32_nearest(total / kblock.shape[0])


# --------------------------------------------------------------------------
# selection keys, certified in float64 with exact fallback
# --------------------------------------------------------------------------


def _certify(y: np.ndarray, e: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    lo = (y - e).astype(np.float32)
    hi = (y + e).astype(np.float32)
    ok = lo == hi
    return (lo + np.float32(0.0)), ok          # + 0.0 turns -0 into +0


def keys_dot(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """key(j) = nearest float32 of q . K[j] (exact real), for every row of K."""
    n, d = K.shape
    if n == 0:
        return np.zeros(0, np.float32)
    y = K @ q
    A = np.abs(K) @ np.abs(q)
    e = 2.0 * (d + 4) * U52 * A + 1e-300
    keys, ok = _certify(y, e)
    for j in np.nonzero(~ok)[0]:
        keys[j] = exact_key_dot(q, K[j])
    return keys


def keys_weighted_relu(Q: np.ndarray, w: np.ndarray, K: np.ndarray) -> np.ndarray:
    """key(j) = nearest float32 of sum_h w_h * max(0, Q[h] . K[j]) (exact real)."""
    n, d = K.shape
    H = Q.shape[0]
    if n == 0:
        return np.zeros(0, np.float32)
    D = K @ Q.T                                   # [n, H]
    A = np.abs(K) @ np.abs(Q).T
    E = 2.0 * (d + 4) * U52 * A + 1e-300
    pos = D > E
    neg = D < -E
    sign_ok = np.all(pos | neg | (w[None, :] == 0), axis=1)
    R = np.where(pos, D, 0.0)
    s = R @ w
    Es = np.where(pos, E, 0.0) @ np.abs(w) + 2.0 * (H + 4) * U52 * (np.abs(R) @ np.abs(w)) + 1e-300
    keys, ok = _certify(s, Es)
    ok &= sign_ok
    for j in np.nonzero(~ok)[0]:
        keys[j] = exact_key_weighted_relu(Q, w, K[j])
    return keys


def keys_blocks(q: np.ndarray, K: np.ndarray, bs: int, n_blocks: int) -> np.ndarray:
    """key(b) = nearest float32 of (1/bs) * sum_{t in block b} q . K[t] (exact real)."""
    d = K.shape[1]
    if n_blocks == 0:
        return np.zeros(0, np.float32)
    Kb = K[: n_blocks * bs].reshape(n_blocks, bs, d)
    ksum = Kb.sum(axis=1)
    kabs = np.abs(Kb).sum(axis=1)
    y = (ksum @ q) / bs
    A = (kabs @ np.abs(q)) / bs
    e = 2.0 * (bs + d + 8) * U52 * A + 1e-300
    keys, ok = _certify(y, e)
    for b in np.nonzero(~ok)[0]:
        keys[b] = exact_key_block(q, Kb[b])
    return keys


# --------------------------------------------------------------------------
# top-K and visible sets
# --------------------------------------------------------------------------


def topk(keys: np.ndarray, K: int) -> np.ndarray:
    """Indices of the min(K, n) largest keys, ties to the lower index; ascending."""
    n = keys.shape[0]
    kk = min(K, n)
    order = np.lexsort((np.arange(n), -keys.astype(np.float64)))
    return np.sort(order[:kk]).astype(np.int32)


def window_global_set(p: int, w: int, g: int, stride: int = 0) -> np.ndarray:
    """Keys j <= p with j >= p - w + 1 (window incl. self), j < g (global) or,
    when stride > 0, j a multiple of stride (dilated stride)."""
    win = np.arange(max(0, p - w + 1), p + 1)
    glob = np.arange(0, min(g, p + 1))
    s = np.union1d(win, glob)
    if stride > 0:
        s = np.union1d(s, np.arange(0, p + 1, stride))
    return s.astype(np.int32)


def eligible_blocks(p: int, bs: int) -> int:
    """Complete past blocks: block b is eligible when its last key bs*b+bs-1 <= p."""
    return (p + 1) // bs


def block_select(q: np.ndarray, K: np.ndarray, p: int, bs: int, nb: int) -> np.ndarray:
    ne = eligible_blocks(p, bs)
    keys = keys_blocks(q, K, bs, ne)
    return topk(keys, nb)


def blocks_set(blocks: Sequence[int], p: int, bs: int, w: int) -> np.ndarray:
    parts = [np.arange(bs * b, bs * b + bs) for b in blocks]
    parts.append(np.arange(max(0, p - w + 1), p + 1))
    s = np.unique(np.concatenate(parts)) if parts else np.zeros(0, np.int64)
    return s[s <= p].astype(np.int32)


def page_keys(keys: np.ndarray, P: int, n_pages: int) -> np.ndarray:
    """key(page) = the largest key among the page's tokens.

    ``keys`` holds the keys of the visible tokens 0..p; page pi covers tokens
    pi*P .. pi*P+P-1, cut at p ("Sparse Attention in 2026", DSA list: one
    rating per 64-token page).
    """
    out = np.empty(n_pages, dtype=np.float32)
    for pi in range(n_pages):
        out[pi] = keys[pi * P:min((pi + 1) * P, keys.shape[0])].max()
    return out


def page_select(keys: np.ndarray, p: int, P: int, top_pages: int, n_local: int) -> np.ndarray:
    """Pages read by the query at position p, ascending.

    The n_local most recent pages (the page holding p and the ones before it)
    are always read; among the earlier pages the min(top_pages, count) best by
    (page key descending, page index ascending) are added ("Sparse Attention
    in 2026", DSA list: top-k relevant pages plus mandatory recent/local pages).
    """
    last = p // P
    n_cand = max(0, last + 1 - n_local)
    chosen = topk(page_keys(keys[:p + 1], P, n_cand), top_pages) if n_cand else np.zeros(0, np.int32)
    local = np.arange(n_cand, last + 1)
    return np.concatenate([chosen, local]).astype(np.int32)


def two_level_select(block_keys: np.ndarray, token_keys: np.ndarray, p: int, bs: int, top_blocks: int,
                     K: int) -> np.ndarray:
    """Positions chosen by the two-level selection at query position p, ascending.

    block_keys: keys of the complete blocks 0..(p+1)//bs - 1; token_keys: keys
    of the tokens 0..p."""
    nbe = (p + 1) // bs
    blocks = topk(block_keys[:nbe], top_blocks)
    cand = np.concatenate([np.arange(bs * b, bs * b + bs) for b in blocks] + [np.arange(nbe * bs, p + 1)])
    cand = np.sort(cand).astype(np.int64)
    chosen = topk(token_keys[cand], K)               # indices into cand, ascending = positions ascending
    return cand[chosen].astype(np.int32)


def quest_bounds(K: np.ndarray, P: int, n_pages: int) -> Tuple[np.ndarray, np.ndarray]:
    """Channel-wise minimum and maximum of the keys of pages 0..n_pages-1
    (each page the P rows pi*P .. pi*P+P-1 of K), each [n_pages, d]."""
    Kp = K[: n_pages * P].reshape(n_pages, P, K.shape[1])
    return Kp.min(axis=1), Kp.max(axis=1)


def exact_quest_key(Q: np.ndarray, mn: np.ndarray, mx: np.ndarray) -> np.float32:
    """Nearest float32 of sum_h sum_c max(Q[h,c] mn[c], Q[h,c] mx[c]), exact rationals."""
    total = Fraction(0)
    for h in range(Q.shape[0]):
        for c in range(Q.shape[1]):
            a = _frac(Q[h, c])
            total += max(a * _frac(mn[c]), a * _frac(mx[c]))
    return f32_nearest(total)


def quest_page_keys(Q: np.ndarray, K: np.ndarray, P: int, n_pages: int) -> np.ndarray:
    """key(page) for the query heads Q [H, d] of one selection group over the
    complete pages 0..n_pages-1 of K: the float32 nearest to the exact bound
    (products of bf16/f32 values are exact in float64; the float64 sum is
    certified against its rounding bound, else summed exactly)."""
    if n_pages == 0:
        return np.zeros(0, np.float32)
    mn, mx = quest_bounds(K, P, n_pages)
    T = np.maximum(Q[None, :, :] * mn[:, None, :], Q[None, :, :] * mx[:, None, :])    # [pages, H, d]
    T = T.reshape(n_pages, -1)
    y = T.sum(axis=1)
    A = np.abs(T).sum(axis=1)
    e = 2.0 * (T.shape[1] + 4) * U52 * A + 1e-300
    keys, ok = _certify(y, e)
    for i in np.nonzero(~ok)[0]:
        keys[i] = exact_quest_key(Q, mn[i], mx[i])
    return keys


def quest_select(Q: np.ndarray, K: np.ndarray, p: int, P: int, top_pages: int, n_local: int) -> np.ndarray:
    """Pages read by the query heads Q [H, d] of one group at position p, ascending:
    the n_local (>= 1) most recent pages, and among the earlier (complete)
    pages the min(top_pages, count) best by (bound key descending, page
    ascending)."""
    assert n_local >= 1
    last = p // P
    n_cand = max(0, last + 1 - n_local)
    chosen = topk(quest_page_keys(Q, K[:p + 1], P, n_cand), top_pages) if n_cand else np.zeros(0, np.int32)
    local = np.arange(n_cand, last + 1)
    return np.concatenate([chosen, local]).astype(np.int32)


def group_block_select(block_keys: np.ndarray, p: int, bs: int, top_blocks: int) -> np.ndarray:
    """Blocks one GQA group reads at position p: the min(top_blocks, count)
    complete past blocks best by (block key descending, block ascending),
    ascending. block_keys: the keys of blocks 0..(p+1)//bs - 1 at least."""
    return topk(block_keys[:(p + 1) // bs], top_blocks)


def pages_set(pages: Sequence[int], p: int, P: int) -> np.ndarray:
    """Every token of the listed pages, within 0..p (pages are read whole)."""
    parts = [np.arange(P * pg, P * pg + P) for pg in pages]
    s = np.unique(np.concatenate(parts)) if len(parts) else np.zeros(0, np.int64)
    return s[s <= p].astype(np.int32)


def pooled_blocks(X: np.ndarray, bs: int, n_blocks: int, fmt: Optional[str] = None) -> np.ndarray:
    """Mean of each complete block of bs rows (the compressed entries), summed
    with math.fsum (correctly rounded) and, with fmt "f32", rounded once to
    the nearest float32 (the indexer's per-block key cache)."""
    out = np.empty((n_blocks, X.shape[1]))
    for b in range(n_blocks):
        for c in range(X.shape[1]):
            out[b, c] = math.fsum(X[b * bs:(b + 1) * bs, c]) / bs
    if fmt is None:
        return out
    if fmt != "f32":
        raise ValueError(fmt)
    return out.astype(np.float32).astype(np.float64)


def nsa_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, p: int, bs: int, blocks: Sequence[int], w: int,
                  gates: np.ndarray, scale: float,
                  pooled: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> np.ndarray:
    """Gated sum of the compression, selection and window branches for one
    query head q [d] at position p (keys K, V [>= p+1, d]); gates [3];
    pooled: the block means already formed (of at least the complete blocks
    up to p)."""
    out = np.zeros(K.shape[1])
    nc = eligible_blocks(p, bs)
    branches = []
    if nc:
        Kc, Vc = pooled if pooled is not None else (pooled_blocks(K, bs, nc), pooled_blocks(V, bs, nc))
        branches.append((0, Kc[:nc], Vc[:nc], np.arange(nc)))
    sel = blocks_set(blocks, p, bs, 0)
    if len(sel):
        branches.append((1, K[: p + 1], V[: p + 1], sel))
    branches.append((2, K[: p + 1], V[: p + 1], window_global_set(p, w, 0)))
    for gi, Kx, Vx, S in branches:
        o, _ = masked_attention(q[None, :], Kx, Vx, S, scale)
        out += gates[gi] * o[0]
    return out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------


def masked_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray,
                     scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Dense masked attention over candidate keys K[0..n) with visible set S.

    q [H, d]; K, V [n, d]; returns O [H, d] and LSE [H] (natural log).
    """
    z = (q @ K.T) * scale                        # [H, n]
    mask = np.zeros(K.shape[0], dtype=bool)
    mask[S] = True
    z = np.where(mask[None, :], z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    O = (e @ V) / l
    lse = (m + np.log(l))[:, 0]
    return O, lse


def masked_attention_grads(q: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray, scale: float,
                           dO: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of sum(dO * O) for O = masked_attention(q, K, V, S).

    q, dO [H, d] (heads that share K and V and the visible set); K, V [n, d].
    With P the masked softmax: dV = P^T dO, dP = dO V^T, D = rowsum(dO * O),
    dS = P * (dP - D), dq = scale dS K, dK = scale dS^T q ("Sparse Attention
    in 2026", natively trainable sparsity: the backward runs over the same
    visible set). An empty visible set has zero gradients.
    """
    H, n = q.shape[0], K.shape[0]
    if len(S) == 0:
        return np.zeros_like(q), np.zeros((n, K.shape[1])), np.zeros((n, V.shape[1]))
    z = (q @ K.T) * scale
    mask = np.zeros(n, dtype=bool)
    mask[S] = True
    z = np.where(mask[None, :], z, -np.inf)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    P = e / e.sum(axis=1, keepdims=True)
    O = P @ V
    dV = P.T @ dO
    dP = dO @ V.T
    D = (dO * O).sum(axis=1, keepdims=True)
    dS = P * (dP - D)
    return scale * dS @ K, scale * dS.T @ q, dV


def softmax_rows(q: np.ndarray, K: np.ndarray, S: np.ndarray, scale: float) -> np.ndarray:
    """The masked softmax probabilities (for checking that rows sum to one)."""
    z = (q @ K.T) * scale
    mask = np.zeros(K.shape[0], dtype=bool)
    mask[S] = True
    z = np.where(mask[None, :], z, -np.inf)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# workload driver
# --------------------------------------------------------------------------


class Rows:
    """Oracle results for a list of (request, query row) pairs."""

    def __init__(self) -> None:
        self.sets: Dict[Tuple[int, int, int], np.ndarray] = {}      # (b, group, r) -> S
        self.keys: Dict[Tuple[int, int, int], np.ndarray] = {}      # token/block keys
        self.blocks: Dict[Tuple[int, int, int], np.ndarray] = {}    # (b, head or group, r) -> blocks or pages
        self.O: Dict[Tuple[int, int], np.ndarray] = {}              # (b, r) -> [Hq, d]
        self.lse: Dict[Tuple[int, int], np.ndarray] = {}
        self.pairs = 0
        self.candidates = 0


def run(wl, inp: Dict[str, np.ndarray], rows: Iterable[Tuple[int, int]],
        attention: bool = True, keep_keys: bool = False) -> Rows:
    """Run the full hot path for the given (request, query row) pairs.

    ``wl`` is a workload description (attributes as in the input generator:
    kind, Hq, Hkv, d, dtype, H_I, G_sel, score_mode, topk, window, ...).
    """
    res = Rows()
    ctx = np.asarray(inp["ctx_len"]).astype(np.int64)
    Q = inp["q"]
    Kst = inp["k"]
    Vst = inp["v"]
    scale = 1.0 / math.sqrt(wl.d)
    qpk = wl.Hq // wl.Hkv
    for (b, r) in rows:
        L = int(ctx[b])
        p = L - wl.Nq + r
        n = p + 1
        Kb = [decode(Kst[b, h, :n], wl.dtype) for h in range(wl.Hkv)]
        # visible set per query head
        S_of_head: List[np.ndarray] = [None] * wl.Hq
        if wl.kind == "msa":
            qi = decode(inp["q_idx"][b, r], wl.idx_q_dtype)
            hpg = wl.H_I // wl.G_sel
            w = np.asarray(inp["w"], dtype=np.float32).astype(np.float64)
            nbe = n // wl.block_size
            for g in range(wl.G_sel):
                kg = g if wl.G_k == wl.G_sel else 0
                Kp = pooled_blocks(decode(inp["k_idx"][b, :nbe * wl.block_size, kg], wl.idx_k_dtype),
                                   wl.block_size, nbe, "f32")
                if wl.score_mode == "dot":
                    bkeys = keys_dot(qi[g * hpg], Kp)
                else:
                    bkeys = keys_weighted_relu(qi[g * hpg:(g + 1) * hpg], w[g * hpg:(g + 1) * hpg], Kp)
                blk = group_block_select(bkeys, p, wl.block_size, wl.top_blocks)
                res.blocks[(b, g, r)] = blk
                if keep_keys:
                    res.keys[(b, g, r)] = bkeys
                S = blocks_set(blk, p, wl.block_size, wl.window)
                res.sets[(b, g, r)] = S
                for h in range(g * (wl.Hq // wl.G_sel), (g + 1) * (wl.Hq // wl.G_sel)):
                    S_of_head[h] = S
        elif wl.kind in ("topk", "dsa_prefill", "dsa_decode", "dsa_pages", "dsa_two_level"):
            qi = decode(inp["q_idx"][b, r], wl.idx_q_dtype)            # [H_I, d_I]
            hpg = wl.H_I // wl.G_sel
            w = np.asarray(inp["w"], dtype=np.float32).astype(np.float64)
            for g in range(wl.G_sel):
                kg = g if wl.G_k == wl.G_sel else 0
                Ki = decode(inp["k_idx"][b, :n, kg], wl.idx_k_dtype)
                if wl.score_mode == "dot":
                    keys = keys_dot(qi[g * hpg], Ki)
                else:
                    keys = keys_weighted_relu(qi[g * hpg:(g + 1) * hpg], w[g * hpg:(g + 1) * hpg], Ki)
                if wl.kind == "dsa_pages":
                    pg = page_select(keys, p, wl.page_size, wl.top_pages, wl.n_local)
                    res.blocks[(b, g, r)] = pg
                    S = pages_set(pg, p, wl.page_size)
                elif wl.kind == "dsa_two_level":
                    nbe = n // wl.block_size
                    Kp = pooled_blocks(Ki, wl.block_size, nbe, "f32")
                    if wl.score_mode == "dot":
                        bkeys = keys_dot(qi[g * hpg], Kp)
                    else:
                        bkeys = keys_weighted_relu(qi[g * hpg:(g + 1) * hpg], w[g * hpg:(g + 1) * hpg], Kp)
                    S = two_level_select(bkeys, keys, p, wl.block_size, wl.top_blocks, wl.topk)
                else:
                    S = topk(keys, wl.topk)
                res.sets[(b, g, r)] = S
                if keep_keys:
                    res.keys[(b, g, r)] = keys
                for h in range(wl.Hq):
                    if h // (wl.Hq // wl.G_sel) == g:
                        S_of_head[h] = S
        elif wl.kind == "quest":
            hg = wl.Hq // wl.G_sel
            for g in range(wl.G_sel):
                Qg = np.stack([decode(Q[b, h, r], wl.dtype) for h in range(g * hg, (g + 1) * hg)])
                pg = quest_select(Qg, Kb[(g * hg) // qpk], p, wl.page_size, wl.top_pages, wl.n_local)
                res.blocks[(b, g, r)] = pg
                S = pages_set(pg, p, wl.page_size)
                res.sets[(b, g, r)] = S
                for h in range(g * hg, (g + 1) * hg):
                    S_of_head[h] = S
        elif wl.kind == "window_global":
            S = window_global_set(p, wl.window, wl.n_global, wl.stride)
            res.sets[(b, 0, r)] = S
            S_of_head = [S] * wl.Hq
        elif wl.kind in ("blocks", "nsa"):
            for h in range(wl.Hq):
                qh = decode(Q[b, h, r], wl.dtype)
                ne = eligible_blocks(p, wl.block_size)
                keys = keys_blocks(qh, Kb[h // qpk], wl.block_size, ne)
                blk = topk(keys, wl.top_blocks)
                res.blocks[(b, h, r)] = blk
                if keep_keys:
                    res.keys[(b, h, r)] = keys
                S = blocks_set(blk, p, wl.block_size, 0 if wl.kind == "nsa" else wl.window)
                res.sets[(b, h, r)] = S
                S_of_head[h] = S
        elif wl.kind == "dense":
            S = np.arange(n, dtype=np.int32)
            res.sets[(b, 0, r)] = S
            S_of_head = [S] * wl.Hq
        else:
            raise ValueError(wl.kind)
        res.candidates += n * wl.Hq
        res.pairs += sum(len(s) for s in S_of_head)
        if attention and wl.kind == "nsa":
            O = np.zeros((wl.Hq, wl.d))
            gates = np.asarray(inp["gates"], dtype=np.float32).astype(np.float64)
            nc = eligible_blocks(p, wl.block_size)
            for kvh in range(wl.Hkv):
                Vh = decode(Vst[b, kvh, :n], wl.dtype)
                pooled = (pooled_blocks(Kb[kvh], wl.block_size, nc), pooled_blocks(Vh, wl.block_size, nc))
                for h in range(kvh * qpk, (kvh + 1) * qpk):
                    qh = decode(Q[b, h, r], wl.dtype)
                    O[h] = nsa_attention(qh, Kb[kvh], Vh, p, wl.block_size, res.blocks[(b, h, r)], wl.window,
                                         gates[b, h, r], scale, pooled=pooled)
            res.O[(b, r)] = O
        elif attention:
            O = np.zeros((wl.Hq, wl.d))
            lse = np.zeros(wl.Hq)
            for h in range(wl.Hq):
                qh = decode(Q[b, h, r], wl.dtype)[None, :]
                kvh = h // qpk
                Vh = decode(Vst[b, kvh, :n], wl.dtype)
                o, l = masked_attention(qh, Kb[kvh], Vh, S_of_head[h], scale)
                O[h] = o[0]
                lse[h] = l[0]
            res.O[(b, r)] = O
            res.lse[(b, r)] = lse
    return res

