"""Seeded synthetic inputs for selective sparse attention workloads.

This module only draws random numbers and encodes them into the storage
formats the library reads (fp32, bf16, fp8-e4m3fn). It holds none of the
method's arithmetic: no scores, no selection, no softmax. Both the CPU oracle
and the GPU path are fed from here, and nothing else is shared between them.

Recipe (stated once, used everywhere):
  * every tensor is drawn from NumPy's PCG64 with
    ``SeedSequence([seed, tensor_id, chunk])`` over chunks of 2**22 elements,
    sampled as float32 N(0,1) (``standard_normal``) or U(0,1) for indexer
    weights, then rounded to nearest-even into bf16 or fp8-e4m3fn;
  * queries are the last ``Nq`` positions of each request's context;
  * "needle" keys (retrieval-style workloads of the DSA/indexer pages) are
    planted on the indexer key only: a key j is replaced by a vector of
    4x its own norm pointing along the unit direction of one query i > j
    (for several indexer heads: the head with the largest weight);
  * the block-sparse workload shifts every key element of 4% of the 64-token
    blocks by +2.0 (two standard deviations) before rounding, the same blocks
    for every head (the NSA workload too);
  * NSA branch gates are U(0,1) draws, one per (request, head, row, branch);
  * decode lengths are drawn uniformly from an inclusive integer range;
  * paged workloads also store K and V as a pool of P-token pages: the
    B * ceil(N/P) logical pages are placed at the physical slots of one seeded
    permutation (page_table[b, page] = slot), so consecutive pages of a
    request are scattered over the pool.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

CHUNK = 1 << 22

# tensor ids used in the seed sequence
TID = dict(q=1, k=2, v=3, q_idx=4, k_idx=5, w=6, lengths=7, needles=8, shift=9, pages=10, gates=11, d_o=12)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------
# storage encodings
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3fn_table() -> np.ndarray:
    """Values of the 256 OCP fp8 E4M3FN codes (bias 7, no infinities, 0x7F/0xFF NaN)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3FN_VALUES = _e4m3fn_table()
_POS_CODES = np.arange(0, 0x7F)           # finite non-negative codes, increasing value
_POS_VALUES = E4M3FN_VALUES[_POS_CODES]


def f32_to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to fp8 E4M3FN (nearest, ties to even code); uint8 codes.

    Magnitudes above the largest finite value (448) are rejected: the
    synthetic workloads never produce them.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    if a.size and a.max() > 448.0:
        raise ValueError("value out of fp8 e4m3fn range")
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    vhi = _POS_VALUES[hi]
    vlo = _POS_VALUES[lo]
    dhi = vhi - a
    dlo = a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0))
    pick_hi |= (vhi == a)
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return code


def e4m3fn_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return E4M3FN_VALUES[np.asarray(b, dtype=np.uint8)].astype(np.float32)


ENCODERS = {
    "f32": lambda x: np.asarray(x, dtype=np.float32),
    "bf16": f32_to_bf16_bits,
    "fp8": f32_to_e4m3fn_bits,
}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def decode(a: np.ndarray, fmt: str) -> np.ndarray:
    """Storage array -> float32 values (exact for all three formats)."""
    if fmt == "f32":
        return np.asarray(a, dtype=np.float32)
    if fmt == "bf16":
        return bf16_bits_to_f32(a)
    if fmt == "fp8":
        return e4m3fn_bits_to_f32(a)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------
def _rng(seed: int, tid: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def normal(seed: int, tid: int, shape, fmt: str, shift_fn=None) -> np.ndarray:
    """N(0,1) float32 draws encoded into ``fmt``; chunked and multi-threaded.

    ``shift_fn(flat_start, values)`` may modify a float32 chunk in place before
    rounding (used for the block-sparse mean shift).
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORAGE[fmt])
    enc = ENCODERS[fmt]
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(ci: int) -> None:
        s = ci * CHUNK
        e = min(n, s + CHUNK)
        buf = np.empty(e - s, dtype=np.float32)
        _rng(seed, tid, ci).standard_normal(out=buf, dtype=np.float32)
        if shift_fn is not None:
            shift_fn(s, buf)
        out[s:e] = enc(buf)

    if nchunks <= 1:
        for ci in range(nchunks):
            work(ci)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def uniform01(seed: int, tid: int, shape) -> np.ndarray:
    return _rng(seed, tid).random(size=shape, dtype=np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # topk | window_global | blocks | nsa | dsa_prefill | dsa_decode | dsa_pages |
                              # dsa_two_level | quest | msa
    B: int
    Hq: int
    Hkv: int
    N: int                    # context capacity (keys per request)
    Nq: int                   # query rows per request (last Nq positions)
    d: int
    dtype: str                # f32 | bf16 (Q, K, V)
    seed: int
    # indexer / token top-K
    H_I: int = 0
    d_I: int = 0
    G_sel: int = 1            # selection groups (index sets per query row)
    G_k: int = 1              # indexer key heads (1 = shared by all groups)
    idx_q_dtype: str = "f32"
    idx_k_dtype: str = "f32"
    score_mode: str = "dot"   # dot | weighted_relu
    topk: int = 0
    needles: int = 0
    # fixed patterns
    window: int = 0
    n_global: int = 0
    stride: int = 0           # dilated stride: every stride-th token is visible too
    block_size: int = 0
    top_blocks: int = 0
    shift_frac: float = 0.0
    shift: float = 0.0
    # page-granular selection over a paged KV cache (dsa_pages, quest; for quest G_sel is
    # the number of page lists per row, H_kv | G_sel | H_q)
    page_size: int = 0
    top_pages: int = 0
    n_local: int = 0
    # backward: an upstream gradient dO is drawn and the gradients are computed
    backward: bool = False
    # decode lengths (inclusive range); None = every request has N keys
    len_range: Optional[Tuple[int, int]] = None

    @property
    def heads_per_group(self) -> int:
        return self.H_I // self.G_sel if self.G_sel else 0


WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


# The five workloads of the selective-sparse-attention hot path.
TINY = _add(Workload("tiny_topk_f32", "topk", B=1, Hq=1, Hkv=1, N=1024, Nq=1024, d=64,
                     dtype="f32", seed=1, H_I=1, d_I=32, G_sel=1, idx_q_dtype="f32",
                     idx_k_dtype="f32", score_mode="dot", topk=64, needles=8))
WINDOW = _add(Workload("window_global", "window_global", B=1, Hq=8, Hkv=8, N=16384,
                       Nq=16384, d=128, dtype="bf16", seed=2, window=512, n_global=16))
BLOCKS = _add(Workload("block_sparse", "blocks", B=1, Hq=16, Hkv=16, N=32768, Nq=32768,
                       d=128, dtype="bf16", seed=3, block_size=64, top_blocks=16,
                       window=512, shift_frac=0.04, shift=2.0))
PREFILL = _add(Workload("dsa_prefill", "dsa_prefill", B=1, Hq=16, Hkv=1, N=65536,
                        Nq=65536, d=128, dtype="bf16", seed=4, H_I=4, d_I=64, G_sel=1,
                        idx_q_dtype="bf16", idx_k_dtype="bf16", score_mode="weighted_relu",
                        topk=2048, needles=655))
DECODE = _add(Workload("dsa_decode", "dsa_decode", B=8, Hq=32, Hkv=8, N=131072, Nq=1,
                       d=128, dtype="bf16", seed=5, H_I=32, d_I=64, G_sel=8, G_k=1,
                       idx_q_dtype="bf16", idx_k_dtype="fp8", score_mode="weighted_relu",
                       topk=2048, len_range=(98304, 131072)))

# Reduced shapes with the same structure (for oracle-speed parity tests).
_add(dataclasses.replace(TINY, name="tiny_topk_f32_small", N=300, Nq=300, needles=3))
_add(dataclasses.replace(WINDOW, name="window_global_small", Hq=2, Hkv=2, N=1000,
                         Nq=1000, window=96, n_global=5))
# Local window plus dilated stride (the fixed pattern's defaults: 64 positions
# back, i.e. 65 keys with the query, and every 8th token).
STRIDED = _add(dataclasses.replace(WINDOW, name="window_stride", seed=8, window=65, n_global=0, stride=8))
# Backward over the window + global pattern (a training step's attention).
_add(dataclasses.replace(WINDOW, name="window_global_bwd", seed=11, Hq=8, Hkv=8, N=4096, Nq=4096, window=256,
                         n_global=16, backward=True))
_add(dataclasses.replace(WINDOW, name="window_global_bwd_small", seed=11, Hq=4, Hkv=2, N=300, Nq=300, window=40,
                         n_global=3, backward=True))
_add(dataclasses.replace(STRIDED, name="window_stride_small", Hq=2, Hkv=2, N=1000, Nq=1000, stride=24,
                         n_global=3))
_add(Workload("dense_small", "dense", B=2, Hq=4, Hkv=2, N=700, Nq=700, d=128, dtype="bf16", seed=6))
_add(dataclasses.replace(BLOCKS, name="block_sparse_small", Hq=2, Hkv=2, N=1500,
                         Nq=1500, top_blocks=4, window=100))
# Three-branch NSA attention on the block-sparse shapes: compression over the
# mean-pooled 64-token blocks, selection of the top-16 blocks, a 512-token
# window, and one gate value per branch for every (row, head).
NSA = _add(dataclasses.replace(BLOCKS, name="nsa_blocks", kind="nsa", seed=9))
_add(dataclasses.replace(NSA, name="nsa_blocks_small", Hq=4, Hkv=2, N=1500, Nq=1500, top_blocks=4, window=100))
_add(dataclasses.replace(PREFILL, name="dsa_prefill_small", Hq=16, N=1200, Nq=1200,
                         topk=128, needles=12))
_add(dataclasses.replace(DECODE, name="dsa_decode_small", B=3, N=9000,
                         topk=512, len_range=(6000, 9000)))

# Page-granular selection over a paged KV cache: the decode shape above with
# 64-token pages, the 30 best pages plus the 2 most recent (2048 tokens read).
PAGED = _add(dataclasses.replace(DECODE, name="dsa_paged_decode", kind="dsa_pages", seed=7,
                                 topk=0, page_size=64, top_pages=30, n_local=2))
_add(dataclasses.replace(PAGED, name="dsa_paged_decode_small", B=3, N=9000, top_pages=6,
                         len_range=(6000, 9000)))
# Two-level selection on the decode shapes: the 64 best 64-token blocks by
# their mean indexer key (about 4K candidate tokens), then the top-2048 tokens.
TWO = _add(dataclasses.replace(DECODE, name="dsa_two_level_decode", kind="dsa_two_level", seed=10,
                               block_size=64, top_blocks=64))
_add(dataclasses.replace(TWO, name="dsa_two_level_decode_small", B=3, N=9000, topk=512, top_blocks=16,
                         len_range=(6000, 9000)))
_add(dataclasses.replace(TWO, name="dsa_two_level_prefill_small", B=1, Hq=8, Hkv=2, N=700, Nq=700, H_I=4,
                         G_sel=2, idx_k_dtype="bf16", block_size=16, top_blocks=6, topk=40, len_range=None))
_add(dataclasses.replace(PAGED, name="dsa_paged_prefill_small", B=1, Hq=8, Hkv=2, N=700, Nq=700,
                         H_I=4, G_sel=2, idx_k_dtype="bf16", page_size=16, top_pages=5,
                         n_local=1, len_range=None))
# Blockwise selection per GQA group (MSA-style) on the block-sparse prefill
# shapes with four KV groups: an 8-head indexer (two heads per group) rates
# each complete 64-token block by its mean indexer key, each group keeps its
# 16 best blocks, and every head of the group attends over them plus a
# 512-token window.
MSA = _add(Workload("msa_prefill", "msa", B=1, Hq=16, Hkv=4, N=32768, Nq=32768, d=128, dtype="bf16", seed=13,
                    H_I=8, d_I=64, G_sel=4, G_k=1, idx_q_dtype="bf16", idx_k_dtype="bf16",
                    score_mode="weighted_relu", block_size=64, top_blocks=16, window=512))
_add(dataclasses.replace(MSA, name="msa_prefill_small", Hq=4, Hkv=2, N=1500, Nq=1500, H_I=4, G_sel=2,
                         top_blocks=4, window=100))
_add(dataclasses.replace(MSA, name="msa_decode_small", B=3, Hq=8, Hkv=2, N=9000, Nq=1, H_I=4, G_sel=2,
                         idx_k_dtype="fp8", top_blocks=8, window=64, len_range=(6000, 9000)))

# Query-aware page selection with no indexer (Quest's bounds): the decode
# shapes above, one page list per KV group from the group's four query heads,
# the 31 best 64-token pages plus the page holding the query (2048 tokens).
QUEST = _add(dataclasses.replace(DECODE, name="quest_decode", kind="quest", seed=12, H_I=0, d_I=0, G_sel=8,
                                 topk=0, page_size=64, top_pages=31, n_local=1))
_add(dataclasses.replace(QUEST, name="quest_decode_small", B=3, N=9000, top_pages=6, len_range=(6000, 9000)))
_add(dataclasses.replace(QUEST, name="quest_prefill_small", B=1, Hq=8, Hkv=2, N=700, Nq=700, G_sel=8,
                         page_size=16, top_pages=5, n_local=2, len_range=None))


def lengths(w: Workload) -> np.ndarray:
    if w.len_range is None:
        return np.full(w.B, w.N, dtype=np.int32)
    lo, hi = w.len_range
    return _rng(w.seed, TID["lengths"]).integers(lo, hi + 1, size=w.B).astype(np.int32)


def _shift_blocks(w: Workload):
    """Which 64-token blocks get the mean shift (shared by heads), and the shift callback."""
    nb = w.N // w.block_size
    n_shift = int(round(w.shift_frac * nb))
    blocks = np.sort(_rng(w.seed, TID["shift"]).choice(nb, size=n_shift, replace=False))
    mark = np.zeros(nb, dtype=bool)
    mark[blocks] = True
    row = w.d
    per_head = w.N * w.d

    def fn(flat_start: int, buf: np.ndarray) -> None:
        idx = np.arange(flat_start, flat_start + buf.size, dtype=np.int64)
        tok = (idx % per_head) // row
        buf[mark[np.minimum(tok // w.block_size, nb - 1)] & (tok < nb * w.block_size)] += w.shift

    return blocks, fn


def generate(w: Workload) -> Dict[str, np.ndarray]:
    """All inputs of a workload, in storage encodings.

    Keys: q [B,Hq,Nq,d], k, v [B,Hkv,N,d], ctx_len [B] int32; for token top-K
    workloads also q_idx [B,Nq,H_I,d_I], k_idx [B,N,G_k,d_I], w [H_I] float32,
    needles int64 [n,3] (request, query position, key position).
    """
    out: Dict[str, np.ndarray] = {}
    out["ctx_len"] = lengths(w)
    out["q"] = normal(w.seed, TID["q"], (w.B, w.Hq, w.Nq, w.d), w.dtype)
    shift_fn = None
    if w.kind in ("blocks", "nsa") and w.shift_frac > 0:
        blocks, shift_fn = _shift_blocks(w)
        out["shifted_blocks"] = blocks.astype(np.int64)
    out["k"] = normal(w.seed, TID["k"], (w.B, w.Hkv, w.N, w.d), w.dtype, shift_fn)
    out["v"] = normal(w.seed, TID["v"], (w.B, w.Hkv, w.N, w.d), w.dtype)
    if w.H_I:
        out["q_idx"] = normal(w.seed, TID["q_idx"], (w.B, w.Nq, w.H_I, w.d_I), w.idx_q_dtype)
        out["k_idx"] = normal(w.seed, TID["k_idx"], (w.B, w.N, w.G_k, w.d_I), w.idx_k_dtype)
        if w.score_mode == "weighted_relu":
            out["w"] = uniform01(w.seed, TID["w"], (w.H_I,))
        else:
            out["w"] = np.ones(w.H_I, dtype=np.float32)
        out["needles"] = _plant_needles(w, out)
    if w.page_size:
        out["page_table"], out["k_pages"], out["v_pages"] = paged_kv(w, out["k"], out["v"])
    if w.kind == "nsa":
        out["gates"] = uniform01(w.seed, TID["gates"], (w.B, w.Hq, w.Nq, 3))   # compression, selection, window
    if w.backward:
        out["d_o"] = normal(w.seed, TID["d_o"], (w.B, w.Hq, w.Nq, w.d), "f32")
    return out


def paged_kv(w: Workload, k: np.ndarray, v: np.ndarray):
    """page_table int32 [B, ceil(N/P)] and the pools [B*ceil(N/P), Hkv, P, d]."""
    P = w.page_size
    npr = (w.N + P - 1) // P
    slots = _rng(w.seed, TID["pages"]).permutation(w.B * npr).astype(np.int32)
    table = slots.reshape(w.B, npr)
    pad = npr * P - w.N

    def pool(x: np.ndarray) -> np.ndarray:
        if pad:
            x = np.concatenate([x, np.zeros(x.shape[:2] + (pad, x.shape[3]), x.dtype)], axis=2)
        # [B, Hkv, npr, P, d] -> [B*npr, Hkv, P, d] in logical order, then placed at the slots
        logical = x.reshape(w.B, w.Hkv, npr, P, w.d).transpose(0, 2, 1, 3, 4).reshape(w.B * npr, w.Hkv, P, w.d)
        out = np.empty_like(logical)
        out[slots] = logical
        return out

    return table, pool(k), pool(v)


def _plant_needles(w: Workload, t: Dict[str, np.ndarray]) -> np.ndarray:
    """Plant needle indexer keys (see module docstring); returns [n,3] (b, i, j)."""
    if w.needles == 0:
        return np.zeros((0, 3), dtype=np.int64)
    rng = _rng(w.seed, TID["needles"])
    q_all = decode(t["q_idx"], w.idx_q_dtype).astype(np.float64)
    k_store = t["k_idx"]
    head = int(np.argmax(t["w"])) if w.score_mode == "weighted_relu" else 0
    used = set()
    rows = []
    b = 0
    first_pos = w.N - w.Nq
    while len(rows) < w.needles:
        i = int(rng.integers(max(w.topk, first_pos), w.N))
        j = int(rng.integers(0, i))
        if j in used:
            continue
        used.add(j)
        qv = q_all[b, i - first_pos, head]
        qhat = qv / np.linalg.norm(qv)
        kj = decode(k_store[b, j, 0], w.idx_k_dtype).astype(np.float64)
        newk = (4.0 * np.linalg.norm(kj) * qhat).astype(np.float32)
        k_store[b, j, 0] = ENCODERS[w.idx_k_dtype](newk)
        rows.append((b, i, j))
    return np.asarray(rows, dtype=np.int64)
