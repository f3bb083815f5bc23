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
    tokens, overlaps counted once; valid for g <= w <= n."""
    return n * (w + g) - w * (w - 1) // 2 - g * w - g * (g - 1) // 2


def dense_causal_pairs(n: int) -> int:
    return n * (n + 1) // 2
