"""The no-allocation forward attention entry point (workspace in a fixed
per-device array) against the entry point that takes a workspace: the same
kernels, so outputs and LSE must be equal bit for bit, on two calls in a row
(the second smaller), plus its size limit, checked on the host."""
import ctypes

import numpy as np
import pytest
import torch

from fine_grained_top_amd import spattn as S


def _decode_case(seed, B, Hq, Hkv, G, ctx, K, device):
    """Decode-shaped index-list attention: one query per request at the last
    position, per-(request, group) ascending lists of K distinct past keys
    (some rows shorter, -1 padded)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, 1, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, ctx, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, ctx, 128, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    lens = rng.integers(ctx // 2, ctx + 1, size=B).astype(np.int32)
    idx = np.full((B, G, 1, K), -1, np.int32)
    for b in range(B):
        for gg in range(G):
            n = K if (b + gg) % 3 else K - 37
            sel = np.sort(rng.choice(int(lens[b]), size=n, replace=False))
            idx[b, gg, 0, :n] = sel
    to = lambda x: x.to(device)
    return to(q), to(k), to(v), to(torch.from_numpy(lens)), to(torch.from_numpy(idx))


def test_noalloc_rejects_more_than_its_scratch():
    """Routed blocks at block-sparse prefill sizes need far more than the
    fixed array: a clear error before any device is touched (runs without a
    GPU; the tensors are zero-stride descriptors)."""
    cap = S.LIB.spattn_noalloc_scratch_bytes()
    assert cap == 32 << 20
    q = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16).expand(1, 16, 32768, 128)
    blk = torch.zeros(1, 1, 1, 16, dtype=torch.int32).expand(1, 16, 32768, 16)
    o = torch.zeros(1, 1, 1, 128).expand(1, 16, 32768, 128)
    sel = S.selection(S.SEL_BLOCKS, blk, window=512, block_size=64)
    tq, to = S.tensor(q), S.tensor(o)
    need = S.LIB.spattn_sparse_attn_fwd_workspace(ctypes.byref(tq), ctypes.byref(tq), ctypes.byref(sel))
    assert need > cap
    rc = S.LIB.spattn_sparse_attn_fwd_noalloc(ctypes.byref(tq), ctypes.byref(tq), ctypes.byref(tq), None, 0.0,
                                              ctypes.byref(sel), ctypes.byref(to), None, None)
    assert rc == 3
    msg = S.spattn_last_error_message()
    assert "fixed" in msg and str(need) in msg


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    assert torch.cuda.is_available()
    dev = "cuda:0"
    # first call: 4 requests x 4 groups, 1024-entry lists; second: smaller
    for case in ((11, 4, 16, 4, 4, 12000, 1024), (12, 2, 8, 2, 2, 5000, 512)):
        seed, B, Hq, Hkv, G, ctx, K = case
        print(f"[gpu] noalloc case seed={seed} B={B} Hq={Hq} Hkv={Hkv} G={G} ctx={ctx} K={K}", flush=True)
        q, k, v, lens, idx = _decode_case(seed, B, Hq, Hkv, G, ctx, K, dev)
        sel = S.selection(S.SEL_INDEX, idx)
        need = S.LIB.spattn_sparse_attn_fwd_workspace(ctypes.byref(S.tensor(q)), ctypes.byref(S.tensor(k)),
                                                      ctypes.byref(sel))
        assert 0 < need <= S.LIB.spattn_noalloc_scratch_bytes()      # the scratch path is taken
        o_ref = torch.full((B, Hq, 1, 128), float("nan"), device=dev)
        lse_ref = torch.full((B, Hq, 1), float("nan"), device=dev)
        S.spattn_sparse_attn_fwd(q, k, v, lens, 0.0, sel, o_ref, lse_ref)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        S.spattn_sparse_attn_fwd_noalloc(q, k, v, lens, 0.0, sel, o, lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o_ref).all() and torch.isfinite(lse_ref).all()
        assert torch.equal(o, o_ref), float((o - o_ref).abs().max())
        assert torch.equal(lse, lse_ref)
