"""Host-side accounting of bench.py: coverage and pair counts (no GPU).

The selection statistics are checked on hand-sized cases whose counts follow
from the definitions: a window of w keys (self included) plus g global
tokens (completesystemdesign.dev "Sparse Attention", sliding window + global
section), token top-K sets of min(K, p + 1) keys, and blocks of 64 tokens
united with a window.
"""
import os
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fine_grained_top_amd.inputs import Workload  # noqa: E402


class _T:
    """Stands in for a device tensor: .cpu().numpy()."""

    def __init__(self, a):
        self.a = np.asarray(a)

    def cpu(self):
        return self

    def numpy(self):
        return self.a


def test_window_global_coverage_matches_brute_force():
    wl = Workload("w", "window_global", B=1, Hq=2, Hkv=2, N=12, Nq=12, d=64, dtype="bf16", seed=0,
                  window=2, n_global=2)
    st = bench.selection_stats(wl, {"ctx_len": np.array([12])}, SimpleNamespace())
    vis = sum(1 for p in range(12) for j in range(p + 1) if j >= p - 1 or j < 2)
    assert vis == 42                                    # the worked count N=12, w=2, g=2
    assert st["pairs_selected"] == 2 * 42
    assert st["pairs_causal"] == 2 * 78
    assert abs(st["coverage"] + st["skipped_kv_ratio"] - 1.0) < 1e-12


def test_token_topk_coverage_uses_the_counts():
    wl = Workload("d", "dsa_decode", B=2, Hq=8, Hkv=2, N=100, Nq=1, d=64, dtype="bf16", seed=0,
                  H_I=4, d_I=64, G_sel=2, topk=16, len_range=(50, 100))
    inp = {"ctx_len": np.array([50, 10])}
    cnt = np.array([[[16], [16]], [[10], [10]]])       # min(K, p + 1) per (b, g, row)
    st = bench.selection_stats(wl, inp, SimpleNamespace(count=_T(cnt)))
    assert st["pairs_selected"] == (16 + 16 + 10 + 10) * 4      # each group serves 4 query heads
    assert st["pairs_causal"] == (50 + 10) * 8
    assert st["coverage"] == round(st["pairs_selected"] / st["pairs_causal"], 6)


def test_blocks_union_window_counted_once():
    # one row at p = 199, window 10 (keys 190..199), blocks 0 and 2 of 64 tokens:
    # block 2 covers 128..191, overlapping the window on 190, 191
    wl = Workload("b", "blocks", B=1, Hq=1, Hkv=1, N=200, Nq=1, d=64, dtype="bf16", seed=0,
                  block_size=64, top_blocks=2, window=10)
    st = bench.selection_stats(wl, {"ctx_len": np.array([200])}, SimpleNamespace(idx=_T([[[[0, 2]]]])))
    keys = set(range(0, 64)) | set(range(128, 192)) | set(range(190, 200))
    assert st["pairs_selected"] == len(keys)
    assert st["pairs_causal"] == 200
