"""Host-side accounting for the benchmark: memory, pair counts and roofline bytes.

Nothing here runs on the hot path; these are the figures the benchmark prints
next to its measurements.
"""
from __future__ import annotations


def kv_cache_memory_gb(batch: int, ctx: int, kv_dim: int, layers: int,
                       sparsity: float = 0.0, bytes_per_element: int = 2) -> float:
    """KV-cache footprint in GiB when only a (1 - sparsity) share of tokens is kept.

    Two tensors (K and V) per layer, each batch x kept tokens x kv_dim
    ("Sparse Attention Is Reshaping Production AI", KV-cache reduction section).
    """
    kept = ctx * (1.0 - sparsity)
    return 2.0 * batch * kept * kv_dim * layers * bytes_per_element / float(1 << 30)


def window_global_pairs(n: int, w: int, g: int) -> int:
    """Causal (query, key) pairs of a w-key window (including self) plus g global
    tokens, overlaps counted once, for n query positions 0..n-1 (w >= 1, g >= 0).

    Window: sum over p of min(w, p + 1). Globals below the window start
    t = p - w + 1: min(g, t) for t = 0..n-w. With n - w >= g this is the
    closed form n(w + g) - w(w - 1)/2 - g w - g(g - 1)/2."""
    ww = min(w, n)
    win = n * ww - ww * (ww - 1) // 2
    T = n - w
    if T < 0:
        glob = 0
    elif T >= g:
        glob = g * (g - 1) // 2 + g * (T - g + 1)
    else:
        glob = T * (T + 1) // 2
    return win + glob


def window_stride_pairs(n: int, w: int, g: int, stride: int) -> int:
    """Causal pairs of a w-key window plus g global tokens plus every
    stride-th token: the window/global count plus, for each query position p,
    the multiples of stride below both the window start p - w + 1 and outside
    the global prefix (those counted already)."""
    import numpy as np
    base = window_global_pairs(n, w, g)
    if stride <= 0:
        return base
    p = np.arange(n, dtype=np.int64)
    hi = p - w                                      # last key below the window
    lo_m = -(-g // stride)                          # first multiple index at or after g
    cnt = np.where(hi >= 0, hi // stride - lo_m + 1, 0)
    return int(base + np.maximum(cnt, 0).sum())


def dense_causal_pairs(n: int) -> int:
    return n * (n + 1) // 2
