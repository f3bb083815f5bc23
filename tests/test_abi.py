"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before touching a device (no compute calls)."""
import ctypes
import os
import re

import pytest
import torch

from fine_grained_top_amd import spattn as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spattn.h")


def declared_symbols():
    src = open(HEADER).read()
    return re.findall(r"SPATTN_API\s+[\w\s\*]+?\b(spattn_\w+)\s*\(", src)


def test_header_symbols_exported():
    names = declared_symbols()
    assert len(names) >= 11
    lib = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert "gfx950" in S.spattn_version()
    assert S.spattn_status_string(0) == "ok"
    assert S.spattn_status_string(3) == "workspace too small"
    assert S.spattn_status_string(99) == "unknown status"


def _ix(q, k, w, mode, hpg):
    return S.indexer(q, k, w, mode, hpg)


def _call_scores(ix, scores, ws_bytes=4096):
    so = S.tensor(scores)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8)
    return S.LIB.spattn_index_scores(ctypes.byref(ix), None, ctypes.byref(so), None,
                                     ws.data_ptr() if ws_bytes else None, ws_bytes, None)


def test_index_scores_validation():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 64, 1, 64, dtype=torch.uint8)
    w = torch.zeros(1, 4, 8)
    sc = torch.zeros(1, 2, 4, 64)
    ok = _ix(q, k, w, S.SCORE_WEIGHTED_RELU, 4)
    # valid arguments reach the device check (no GPU here)
    assert _call_scores(ok, sc) == 4
    # heads_per_group must divide H_I
    assert _call_scores(_ix(q, k, w, S.SCORE_WEIGHTED_RELU, 3), sc) == 1
    # DOT needs one head per group
    assert _call_scores(_ix(q, k, None, S.SCORE_DOT, 4), sc) == 1
    # f32 queries with fp8 keys is not supported
    assert _call_scores(_ix(q.float(), k, w, S.SCORE_WEIGHTED_RELU, 4), sc) == 2
    # scores shape mismatch
    assert _call_scores(ok, torch.zeros(1, 2, 4, 63)) == 1
    # missing weights in weighted-ReLU mode
    assert _call_scores(_ix(q, k, None, S.SCORE_WEIGHTED_RELU, 4), sc) == 1
    # workspace too small
    assert _call_scores(ok, sc, ws_bytes=0) == 3
    # non-contiguous innermost dim
    qt = torch.zeros(1, 4, 64, 8, dtype=torch.bfloat16).transpose(2, 3)
    assert _call_scores(_ix(qt, k, w, S.SCORE_WEIGHTED_RELU, 4), sc) == 1
    assert "contiguous" in S.spattn_last_error_message()


def test_topk_validation():
    sc = torch.zeros(1, 1, 4, 64)
    io = torch.zeros(1, 1, 4, 8, dtype=torch.int32)

    need = S.LIB.spattn_topk_workspace(ctypes.byref(S.tensor(sc)), None, 8, 0)
    assert 0 < need < (1 << 20)                 # the row kernels' per-row flags
    ws = torch.zeros(need, dtype=torch.uint8)

    def call(k, flags, idx=io, err=None, ix=None, ws_bytes=need):
        s, o = S.tensor(sc), S.tensor(idx)
        return S.LIB.spattn_topk(ctypes.byref(s), err, ix, None, k, flags, ctypes.byref(o), None,
                                 ws.data_ptr(), ws_bytes, None)

    assert call(8, 0) == 4                      # valid: reaches the device check
    assert call(8, 0, ws_bytes=need - 1) == 3   # workspace too small
    assert call(0, 0) == 1                      # K must be >= 1
    assert call(8, 0, idx=torch.zeros(1, 1, 4, 7, dtype=torch.int32)) == 1
    assert call(8, S.TOPK_CERTIFIED) == 1       # certified needs err + indexer
    assert call(8, 1 << 5) == 1                 # unknown flag
    assert call(8, 0, idx=torch.zeros(1, 1, 4, 8, dtype=torch.float32)) == 1


def test_attention_validation():
    q = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16)
    o = torch.zeros(1, 4, 8, 128)
    idx = torch.zeros(1, 2, 8, 4, dtype=torch.int32)

    def call(sel, qq=q, kk=k, vv=k, oo=o, scale=0.0):
        tq, tk, tv, to = S.tensor(qq), S.tensor(kk), S.tensor(vv), S.tensor(oo)
        ws = torch.zeros(1 << 20, dtype=torch.uint8)
        return S.LIB.spattn_sparse_attn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), None, scale,
                                            ctypes.byref(sel), ctypes.byref(to), None, ws.data_ptr(),
                                            ws.numel(), None)

    assert call(S.selection(S.SEL_INDEX, idx)) == 4
    assert call(S.selection(S.SEL_WINDOW_GLOBAL, window=8, n_global=2)) == 4
    assert call(S.selection(S.SEL_WINDOW_GLOBAL, window=8, n_global=2, stride=4)) == 4
    assert call(S.selection(S.SEL_WINDOW_GLOBAL, window=8, stride=-1)) == 1
    assert call(S.selection(S.SEL_DENSE)) == 4
    assert call(S.selection(7)) == 1
    assert call(S.selection(S.SEL_INDEX, idx.float())) == 1
    assert call(S.selection(S.SEL_INDEX, torch.zeros(1, 3, 8, 4, dtype=torch.int32))) == 1   # 3 does not divide 4
    assert call(S.selection(S.SEL_DENSE), qq=torch.zeros(1, 4, 8, 96, dtype=torch.bfloat16),
                kk=torch.zeros(1, 2, 16, 96, dtype=torch.bfloat16),
                vv=torch.zeros(1, 2, 16, 96, dtype=torch.bfloat16), oo=torch.zeros(1, 4, 8, 96)) == 2
    assert call(S.selection(S.SEL_DENSE), kk=torch.zeros(1, 3, 16, 128, dtype=torch.bfloat16)) == 1
    assert call(S.selection(S.SEL_DENSE), scale=float("nan")) == 1
    assert call(S.selection(S.SEL_DENSE), oo=torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)) == 1


def test_block_select_validation():
    q = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    out = torch.zeros(1, 2, 128, 2, dtype=torch.int32)

    def call(bs, nb, oo=out, ws_bytes=1 << 20):
        tq, tk, to = S.tensor(q), S.tensor(k), S.tensor(oo)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8)
        return S.LIB.spattn_block_select(ctypes.byref(tq), ctypes.byref(tk), None, bs, nb, ctypes.byref(to),
                                         None, ws.data_ptr(), ws_bytes, None)

    assert call(16, 2) == 4
    assert call(24, 2) == 1                      # not a power of two
    assert call(16, 0) == 1
    assert call(16, 2, ws_bytes=8) == 3
    assert call(16, 3) == 1                      # output width must equal top_blocks


def test_page_select_validation():
    sc = torch.zeros(1, 2, 4, 256)
    io = torch.zeros(1, 2, 4, 5, dtype=torch.int32)

    ws = torch.zeros(1 << 20, dtype=torch.uint8)

    def call(P, top, loc, flags=0, idx=io, scores=sc, ws_bytes=1 << 20):
        s, o = S.tensor(scores), S.tensor(idx)
        return S.LIB.spattn_page_select(ctypes.byref(s), None, None, None, P, top, loc, flags, ctypes.byref(o),
                                        None, ws.data_ptr(), ws_bytes, None)

    # few rows: the page keys of every row are staged in the workspace
    need = S.LIB.spattn_page_select_workspace(ctypes.byref(S.tensor(sc)), None, 64, 3, 2, 0)
    assert need == 8 * 4 * 4
    assert call(64, 3, 2) == 4                  # valid: reaches the device check
    assert call(64, 3, 2, ws_bytes=need - 1) == 3
    many = torch.zeros(1, 1, 600, 700)          # many rows: one pass per row, no workspace
    assert S.LIB.spattn_page_select_workspace(ctypes.byref(S.tensor(many)), None, 64, 3, 2, 0) == 0
    assert call(16, 5, 0) == 4
    assert call(48, 3, 2) == 1                  # page size not a power of two
    assert call(8192, 3, 2) == 1                # page size above 4096
    assert call(64, 0, 0, idx=torch.zeros(1, 2, 4, 0, dtype=torch.int32)) == 1
    assert call(64, -1, 6) == 1
    assert call(64, 3, 1) == 1                  # width must be top_pages + n_local
    assert call(64, 3, 2, flags=S.TOPK_CERTIFIED) == 1   # certified needs err + indexer
    assert call(64, 3, 2, flags=S.TOPK_FUSED_INDEX) == 1  # fused takes no scores
    assert call(1, 3, 2, scores=torch.zeros(1, 2, 4, 20000)) == 2   # more than 16384 pages
    assert "pages" in S.spattn_last_error_message()


def test_paged_attention_validation():
    q = torch.zeros(2, 4, 1, 128, dtype=torch.bfloat16)
    pool = torch.zeros(6, 2, 16, 128, dtype=torch.bfloat16)
    table = torch.zeros(2, 3, dtype=torch.int32)
    o = torch.zeros(2, 4, 1, 128)
    pidx = torch.zeros(2, 2, 1, 3, dtype=torch.int32)

    def call(sel, kk=pool, vv=pool, tab=table, P=16, oo=o):
        tq, tk, tv, to = S.tensor(q), S.tensor(kk), S.tensor(vv), S.tensor(oo)
        pg = S.kv_pages(tab, P)
        ws = torch.zeros(1 << 20, dtype=torch.uint8)
        return S.LIB.spattn_sparse_attn_fwd_paged(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                                  ctypes.byref(pg), None, 0.0, ctypes.byref(sel), ctypes.byref(to),
                                                  None, ws.data_ptr(), ws.numel(), None)

    assert call(S.selection(S.SEL_PAGES, pidx, block_size=16)) == 4
    assert call(S.selection(S.SEL_INDEX, torch.zeros(2, 2, 1, 8, dtype=torch.int32))) == 4
    assert call(S.selection(S.SEL_DENSE)) == 4
    assert call(S.selection(S.SEL_PAGES, pidx, block_size=12)) == 1            # not a power of two
    assert call(S.selection(S.SEL_PAGES, pidx, block_size=16), P=8) == 1       # pool pages hold 16 tokens
    assert call(S.selection(S.SEL_DENSE), tab=torch.zeros(3, 3, dtype=torch.int32)) == 1   # one row per request
    assert call(S.selection(S.SEL_DENSE), tab=torch.zeros(2, 3)) == 1          # table must be int32
    assert call(S.selection(S.SEL_DENSE), vv=torch.zeros(6, 2, 16, 64, dtype=torch.bfloat16)) == 1
    # the plain entry point is unchanged by the page-list mode
    tq, tk, to = S.tensor(q), S.tensor(torch.zeros(2, 2, 48, 128, dtype=torch.bfloat16)), S.tensor(o)
    sel = S.selection(S.SEL_PAGES, pidx, block_size=16)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    assert S.LIB.spattn_sparse_attn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tk), None, 0.0,
                                        ctypes.byref(sel), ctypes.byref(to), None, ws.data_ptr(), ws.numel(),
                                        None) == 4


def test_page_select_fused_validation():
    q = torch.zeros(2, 1, 32, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 4096, 1, 64, dtype=torch.uint8)
    w = torch.zeros(2, 1, 32)
    ix = S.indexer(q, k, w, S.SCORE_WEIGHTED_RELU, 4)
    io = torch.zeros(2, 8, 1, 5, dtype=torch.int32)
    need = S.LIB.spattn_page_select_workspace(None, ctypes.byref(ix), 64, 3, 2, S.TOPK_FUSED_INDEX)
    rows = 2 * 8
    assert need >= rows * 4096 * 4 + rows * (4096 // 64) * 4   # scores and page keys
    ws = torch.zeros(need, dtype=torch.uint8)

    def call(flags=S.TOPK_FUSED_INDEX, scores=None, ws_bytes=need, idx=io):
        sp_ = ctypes.byref(S.tensor(scores)) if scores is not None else None
        return S.LIB.spattn_page_select(sp_, None, ctypes.byref(ix), None, 64, 3, 2, flags,
                                        ctypes.byref(S.tensor(idx)), None, ws.data_ptr(), ws_bytes, None)

    assert call() == 4                                          # valid: reaches the device check
    assert call(ws_bytes=need - 1) == 3
    assert call(scores=torch.zeros(2, 8, 1, 4096)) == 1         # fused takes no scores
    assert call(idx=torch.zeros(2, 8, 1, 4, dtype=torch.int32)) == 1



def test_nsa_validation():
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 256, 128, dtype=torch.bfloat16)
    blk = torch.zeros(1, 2, 64, 4, dtype=torch.int32)
    gates = torch.zeros(1, 2, 64, 3)
    o = torch.zeros(1, 2, 64, 128)
    need = S.LIB.spattn_nsa_fwd_workspace(ctypes.byref(S.tensor(q)), ctypes.byref(S.tensor(k)), 64,
                                          ctypes.byref(S.tensor(blk)), 32)
    assert need >= 2 * 2 * 4 * 128 * 2 + 3 * 2 * 64 * 128 * 4    # pooled K, V and three branch outputs
    ws = torch.zeros(need, dtype=torch.uint8)

    def call(bs=64, b=blk, g=gates, w=32, ws_bytes=need, oo=o):
        t = [S.tensor(x) for x in (q, k, k, b, g, oo)]
        return S.LIB.spattn_nsa_fwd(ctypes.byref(t[0]), ctypes.byref(t[1]), ctypes.byref(t[2]), None, 0.0, bs,
                                    ctypes.byref(t[3]), w, ctypes.byref(t[4]), ctypes.byref(t[5]), ws.data_ptr(),
                                    ws_bytes, None)

    assert call() == 4
    assert call(bs=48) == 1                       # not a power of two
    assert call(w=-1) == 1
    assert call(g=torch.zeros(1, 2, 64, 2)) == 1  # three gates per row
    assert call(b=torch.zeros(1, 1, 64, 4, dtype=torch.int32)) == 1
    assert call(ws_bytes=need - 1) == 3



def test_two_level_validation():
    q = torch.zeros(2, 1, 32, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 4096, 1, 64, dtype=torch.uint8)
    w = torch.zeros(2, 1, 32)
    ix = S.indexer(q, k, w, S.SCORE_WEIGHTED_RELU, 4)
    kb = torch.zeros(2, 64, 1, 64)
    io = torch.zeros(2, 8, 1, 100, dtype=torch.int32)

    def call(bs=64, nb=8, K=100, blocks=kb, idx=io):
        return S.LIB.spattn_topk_two_level(ctypes.byref(ix), ctypes.byref(S.tensor(blocks)), None, bs, nb, K,
                                           ctypes.byref(S.tensor(idx)), None, None, 0, None)

    assert S.LIB.spattn_topk_two_level_workspace(ctypes.byref(ix), ctypes.byref(S.tensor(kb)), 64, 8, 100) == 0
    assert call() == 4                                    # valid: reaches the device check
    assert call(bs=48) == 1
    assert call(nb=0) == 1
    assert call(nb=200) == 2                              # (top_blocks + 1) * block_size > 8192
    assert call(blocks=torch.zeros(2, 63, 1, 64)) == 1    # fewer block rows than ctx / block_size
    assert call(blocks=kb.to(torch.bfloat16)) == 1        # block keys are f32
    assert call(idx=torch.zeros(2, 8, 1, 99, dtype=torch.int32)) == 1
    assert S.LIB.spattn_pool_index_keys(ctypes.byref(ix), None, 64, ctypes.byref(S.tensor(kb)), None) == 4



def test_backward_validation():
    q = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16)
    o = torch.zeros(1, 4, 8, 128)
    lse = torch.zeros(1, 4, 8)
    dk = torch.zeros(1, 2, 16, 128)

    def call(sel=S.selection(S.SEL_DENSE), oo=o, lp=lse, dkk=dk):
        t = [S.tensor(x) for x in (q, k, k, oo, o, o, dkk, dk)]
        return S.LIB.spattn_sparse_attn_bwd(ctypes.byref(t[0]), ctypes.byref(t[1]), ctypes.byref(t[2]), None, 0.0,
                                            ctypes.byref(sel), ctypes.byref(t[3]), None if lp is None else lp.data_ptr(),
                                            ctypes.byref(t[4]), ctypes.byref(t[5]), ctypes.byref(t[6]),
                                            ctypes.byref(t[7]), None, 0, None)

    assert call() == 4
    assert call(S.selection(S.SEL_WINDOW_GLOBAL, window=4, stride=2)) == 4
    # window pattern on the bf16 tile path: a workspace of slots per band key tile
    qb = torch.zeros(1, 4, 200, 128, dtype=torch.bfloat16)
    kb = torch.zeros(1, 2, 200, 128, dtype=torch.bfloat16)
    selw = S.selection(S.SEL_WINDOW_GLOBAL, window=100, n_global=3)
    need = S.spattn_sparse_attn_bwd_workspace(qb, kb, selw)
    assert need == 1 * 4 * 4 * (100 // 64 + 3) * 64 * 128 * 2 * 4    # B * Hq * key tiles * slots * slot bytes
    assert S.spattn_sparse_attn_bwd_workspace(qb, kb, S.selection(S.SEL_DENSE)) == 0
    tb = [S.tensor(x) for x in (qb, kb, kb, torch.zeros(1, 4, 200, 128), torch.zeros(1, 4, 200, 128),
                                torch.zeros(1, 4, 200, 128), torch.zeros(1, 2, 200, 128), torch.zeros(1, 2, 200, 128))]
    lsew = torch.zeros(1, 4, 200)
    rc = S.LIB.spattn_sparse_attn_bwd(ctypes.byref(tb[0]), ctypes.byref(tb[1]), ctypes.byref(tb[2]), None, 0.0,
                                      ctypes.byref(selw), ctypes.byref(tb[3]), lsew.data_ptr(), ctypes.byref(tb[4]),
                                      ctypes.byref(tb[5]), ctypes.byref(tb[6]), ctypes.byref(tb[7]), None, 0, None)
    assert rc == 3                                                # workspace too small, before any device use
    assert call(lp=None) == 1                                     # the forward's LSE is required
    assert call(oo=torch.zeros(1, 4, 8, 64)) == 1
    assert call(dkk=torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16)) == 1


def test_quest_validation():
    B, Hq, Hkv, Nq, d, maxp, P = 2, 8, 2, 1, 128, 5, 16
    q = torch.zeros(B, Hq, Nq, d, dtype=torch.bfloat16)
    bnd = torch.zeros(B, maxp, Hkv, 2 * d, dtype=torch.bfloat16)
    io = torch.zeros(B, Hkv, Nq, 4, dtype=torch.int32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)

    def sel(top=3, loc=1, P_=P, qq=q, bb=bnd, idx=io, ws_bytes=1 << 20):
        tq, tb, to = S.tensor(qq), S.tensor(bb), S.tensor(idx)
        return S.LIB.spattn_quest_select(ctypes.byref(tq), ctypes.byref(tb), None, P_, top, loc, ctypes.byref(to),
                                         None, ws.data_ptr(), ws_bytes, None)

    need = S.LIB.spattn_quest_select_workspace(ctypes.byref(S.tensor(q)), ctypes.byref(S.tensor(bnd)), P, 3, 1,
                                               ctypes.byref(S.tensor(io)))
    assert need == B * Hkv * Nq * maxp * 4
    assert sel() == 4                                        # valid: reaches the device check
    assert sel(idx=torch.zeros(B, Hq, Nq, 4, dtype=torch.int32)) == 4    # one list per query head
    assert sel(ws_bytes=need - 1) == 3
    assert sel(loc=0, top=4) == 1                            # the query's own page must be read
    assert "n_local" in S.spattn_last_error_message()
    assert sel(top=2) == 1                                   # width must be top_pages + n_local
    assert sel(idx=torch.zeros(B, 3, Nq, 4, dtype=torch.int32)) == 1     # H_kv must divide G
    assert sel(P_=24) == 1                                   # page size not a power of two
    assert sel(bb=torch.zeros(B, maxp, Hkv, d, dtype=torch.bfloat16)) == 1   # bounds need 2d
    assert sel(bb=bnd.float()) == 1                          # bounds in q's dtype
    assert sel(qq=torch.zeros(B, Hq, Nq, 96, dtype=torch.bfloat16),
               bb=torch.zeros(B, maxp, Hkv, 192, dtype=torch.bfloat16)) == 2   # head dim 96
    big = torch.zeros(1, 64, 1, d, dtype=torch.bfloat16)
    assert sel(qq=big, bb=torch.zeros(1, maxp, 2, 2 * d, dtype=torch.bfloat16),
               idx=torch.zeros(1, 2, 1, 4, dtype=torch.int32)) == 2            # 32 heads per group

    pool = torch.zeros(7, Hkv, P, d, dtype=torch.bfloat16)
    table = torch.zeros(B, maxp, dtype=torch.int32)

    def bounds(kk=pool, tab=table, P_=P, bb=bnd):
        pg = S.kv_pages(tab, P_)
        return S.LIB.spattn_quest_page_bounds(ctypes.byref(S.tensor(kk)), ctypes.byref(pg), None,
                                              ctypes.byref(S.tensor(bb)), None)

    assert bounds() == 4
    assert bounds(tab=torch.zeros(B, maxp + 1, dtype=torch.int32)) == 1      # max_pages disagree
    assert bounds(P_=32) == 1                                                 # pool rows are pages of 16
    assert bounds(bb=bnd.float()) == 1                                        # bounds in the key dtype
    assert bounds(bb=torch.zeros(B, maxp, 3, 2 * d, dtype=torch.bfloat16)) == 1   # KV heads disagree


def test_index_block_select_validation():
    B, Nq, ctx, H_I, d_I, bs = 1, 4, 256, 4, 64, 16
    q_idx = torch.zeros(B, Nq, H_I, d_I, dtype=torch.bfloat16)
    k_idx = torch.zeros(B, ctx, 1, d_I, dtype=torch.bfloat16)
    w = torch.zeros(B, Nq, H_I)
    ix = S.indexer(q_idx, k_idx, w, S.SCORE_WEIGHTED_RELU, 2)            # two selection groups
    kb = torch.zeros(B, ctx // bs, 1, d_I)

    def call(top=3, out=None, P=bs, kbl=kb):
        o = torch.zeros(B, 2, Nq, top, dtype=torch.int32) if out is None else out
        return S.LIB.spattn_index_block_select(ctypes.byref(ix), ctypes.byref(S.tensor(kbl)), None, P, top,
                                               ctypes.byref(S.tensor(o)), None, None)

    assert call() == 4                                                   # valid: reaches the device check
    assert call(top=0, out=torch.zeros(B, 2, Nq, 0, dtype=torch.int32)) == 1
    assert call(out=torch.zeros(B, 1, Nq, 3, dtype=torch.int32)) == 1     # one list per selection group
    assert call(out=torch.zeros(B, 2, Nq, 4, dtype=torch.int32)) == 1     # width must be top_blocks
    assert call(P=24) == 1                                               # block size not a power of two
    assert call(kbl=torch.zeros(B, ctx // bs, 1, d_I, dtype=torch.bfloat16)) == 1   # block keys are f32


def test_blocks_selection_groups_validation():
    q = torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    o = torch.zeros(1, 8, 4, 128)

    def call(G):
        blk = torch.zeros(1, G, 4, 3, dtype=torch.int32)
        sel = S.selection(S.SEL_BLOCKS, blk, window=8, block_size=16)
        ws = torch.zeros(1 << 20, dtype=torch.uint8)
        return S.LIB.spattn_sparse_attn_fwd(ctypes.byref(S.tensor(q)), ctypes.byref(S.tensor(k)),
                                            ctypes.byref(S.tensor(k)), None, 0.0, ctypes.byref(sel),
                                            ctypes.byref(S.tensor(o)), None, ws.data_ptr(), ws.numel(), None)

    for G in (1, 2, 4, 8):
        assert call(G) == 4, G                                           # G_sel divides H_q
    assert call(3) == 1
