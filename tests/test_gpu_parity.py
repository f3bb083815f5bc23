"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Index sets must match bit for bit; outputs within max-abs 1e-5 (fp32 inputs)
or 2e-3 (bf16 inputs, fp32 accumulation); LSE within the same bounds.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

from fine_grained_top_amd import inputs as gen

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.init()


def S():
    from fine_grained_top_amd import spattn
    return spattn


def run(wl, inp):
    from fine_grained_top_amd.hotpath import HotPath
    say(f"[gpu] {wl.name}: B={wl.B} N={wl.N} Nq={wl.Nq} Hq={wl.Hq}")
    hp = HotPath(wl, inp)
    hp.step()
    torch.cuda.synchronize()
    return hp


def oracle_rows(wl, inp, rows, attention=True):
    import oracle as orc
    return orc.run(wl, inp, rows, attention=attention)


def check_sets(hp, res, rows, wl):
    idx = hp.idx.cpu().numpy()
    cnt = hp.count.cpu().numpy()
    groups = wl.Hq if wl.kind in ("blocks", "nsa") else wl.G_sel
    listed = wl.kind in ("blocks", "nsa", "dsa_pages", "quest", "msa")   # block or page lists, not token sets
    bad = 0
    for (b, r) in rows:
        for g in range(groups):
            want = res.blocks[(b, g, r)] if listed else res.sets[(b, g, r)]
            got = idx[b, g, r]
            ok = cnt[b, g, r] == len(want) and np.array_equal(got[:len(want)], want) and np.all(got[len(want):] == -1)
            if not ok:
                bad += 1
                if bad <= 3:
                    say(f"  set mismatch b={b} g={g} r={r}: count {cnt[b, g, r]} vs {len(want)}; "
                        f"extra {sorted(set(got[:cnt[b, g, r]]) - set(want))[:8]} missing {sorted(set(want) - set(got))[:8]}")
    assert bad == 0, f"{bad} rows differ"


def check_out(hp, res, rows, tol):
    O = hp.o.cpu().numpy()
    lse = hp.lse.cpu().numpy()
    worst = 0.0
    worst_l = 0.0
    for (b, r) in rows:
        worst = max(worst, float(np.abs(O[b, :, r, :] - res.O[(b, r)]).max()))
        if (b, r) in res.lse:                              # the NSA sum of branches has no single LSE
            worst_l = max(worst_l, float(np.abs(lse[b, :, r] - res.lse[(b, r)]).max()))
    say(f"  max |O - O_oracle| = {worst:.3e}, max |LSE - LSE_oracle| = {worst_l:.3e} (tol {tol})")
    assert worst <= tol and worst_l <= tol


# ---------------------------------------------------------------- layout probes
@pytest.mark.parametrize("kfmt", ["fp8", "bf16"])
def test_indexer_operand_layout_probe(kfmt):
    """One-hot queries read back every element of every key: checks the MFMA
    operand/accumulator layouts and the fp8 -> bf16 conversion."""
    from fine_grained_top_amd.hotpath import to_device
    sp = S()
    say(f"[gpu] layout probe {kfmt}")
    B, Nq, ctx, d = 1, 64, 512, 64
    rng = np.random.default_rng(0)
    qv = np.zeros((B, Nq, 1, d), np.float32)
    for r in range(Nq):
        qv[0, r, 0, r] = 1.0
    if kfmt == "fp8":
        codes = rng.integers(0, 256, size=(B, ctx, 1, d)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x11
        kst = codes
        kval = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    else:
        kf = rng.standard_normal((B, ctx, 1, d)).astype(np.float32)
        kst = gen.f32_to_bf16_bits(kf)
        kval = gen.bf16_bits_to_f32(kst)
    q = to_device(gen.f32_to_bf16_bits(qv), "bf16")
    k = to_device(kst, kfmt)
    ix = sp.indexer(q, k, None, sp.SCORE_DOT, 1)
    scores = torch.full((B, 1, Nq, ctx), float("nan"), device="cuda")
    err = torch.empty(B, 1, Nq, device="cuda")
    sp.spattn_index_scores(ix, None, scores, err)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for r in range(Nq):
        p = ctx - Nq + r
        assert np.array_equal(got[0, 0, r, : p + 1], kval[0, : p + 1, 0, r]), r
    e = err.cpu().numpy()
    assert np.all(e > 0) and np.all(np.isfinite(e))


# ---------------------------------------------------------------- small workloads, every row
def _all_rows(wl, inp):
    return [(b, r) for b in range(wl.B) for r in range(wl.Nq)]


def test_tiny_fp32_full():
    wl = gen.WORKLOADS["tiny_topk_f32"]
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 1e-5)
    idx = hp.idx.cpu().numpy()
    for (b, i, j) in inp["needles"]:
        assert j in idx[b, 0, i]


@pytest.mark.parametrize("name", ["dsa_decode_small", "dsa_prefill_small", "window_global_small",
                                  "block_sparse_small", "tiny_topk_f32_small", "dsa_paged_decode_small",
                                  "dsa_paged_prefill_small", "window_stride_small", "nsa_blocks_small",
                                  "dsa_two_level_decode_small", "dsa_two_level_prefill_small",
                                  "quest_decode_small", "quest_prefill_small", "msa_prefill_small",
                                  "msa_decode_small"])
def test_small_workload(name):
    wl = gen.WORKLOADS[name]
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    if hp.idx is not None:
        check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 1e-5 if wl.dtype == "f32" else 2e-3)


def test_run_twice_is_bitwise_identical():
    wl = gen.WORKLOADS["dsa_decode_small"]
    inp = gen.generate(wl)
    hp = run(wl, inp)
    o1, i1 = hp.o.clone(), hp.idx.clone()
    hp.step()
    torch.cuda.synchronize()
    assert torch.equal(hp.idx, i1)
    assert torch.equal(hp.o, o1)


# ---------------------------------------------------------------- top-K edge cases
def _topk_on(scores_np, K, ctx_len=None, Nq=None):
    sp = S()
    B, G, nq, ctx = scores_np.shape
    sc = torch.from_numpy(scores_np).cuda()
    idx = torch.empty(B, G, nq, K, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, G, nq, dtype=torch.int32, device="cuda")
    cl = None if ctx_len is None else torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    sp.spattn_topk(sc, None, None, cl, K, 0, idx, cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def test_topk_ties_and_edges():
    import oracle as orc
    say("[gpu] top-K ties/edges")
    rng = np.random.default_rng(5)
    B, G, Nq, ctx = 2, 2, 40, 5000
    sc = rng.integers(-4, 5, size=(B, G, Nq, ctx)).astype(np.float32)     # heavy ties
    sc[0, 0] = 1.0                                                        # a row of all-equal
    sc[1, 1, :, ::3] = -0.0
    sc[1, 1, :, 1::3] = 0.0
    ctx_len = [ctx, 3100]
    for K in (1, 7, 2048, 4999, 6000):
        idx, cnt = _topk_on(sc, K, ctx_len)
        for b in range(B):
            for g in range(G):
                for r in range(Nq):
                    p = ctx_len[b] - Nq + r
                    want = orc.topk(sc[b, g, r, : p + 1], K)
                    assert cnt[b, g, r] == len(want)
                    assert np.array_equal(idx[b, g, r, : len(want)], want), (K, b, g, r)
                    assert np.all(idx[b, g, r, len(want):] == -1)


def test_topk_random_long_rows():
    import oracle as orc
    say("[gpu] top-K long rows")
    rng = np.random.default_rng(6)
    sc = rng.standard_normal((1, 4, 2, 131072)).astype(np.float32)
    sc[0, 1] = np.round(sc[0, 1] * 8) / 8        # coarse values: ties at the boundary
    sc[0, 3] = 0.5                               # all equal: too many candidates for the short list
    idx, cnt = _topk_on(sc, 2048)
    for g in range(4):
        for r in range(2):
            p = 131072 - 2 + r
            want = orc.topk(sc[0, g, r, : p + 1], 2048)
            assert np.array_equal(idx[0, g, r], want)


def test_certified_selection_at_rounding_midpoints():
    """Keys whose exact value is a float32 halfway point: the float32 scores tie,
    the exact keys decide (ties to even), then lower index."""
    import oracle as orc
    sp = S()
    say("[gpu] certified midpoints")
    d, ctx, Nq = 8, 64, 1
    q = np.zeros((1, Nq, 1, d), np.float32)
    q[0, 0, 0, :2] = 1.0
    k = np.zeros((1, ctx, 1, d), np.float32)
    rng = np.random.default_rng(7)
    k[0, :, 0, 0] = 1.0
    tiny = np.float32(2.0 ** -24)
    # exact 1 + 2^-24 (rounds to 1.0), 1 + 2^-24 + 2^-40 (rounds up), 1.0, 1 + 3*2^-24 (to 1 + 2^-22)
    pattern = [tiny, tiny + np.float32(2.0 ** -40), 0.0, 3 * tiny]
    for j in range(ctx):
        k[0, j, 0, 1] = pattern[j % 4] if j % 5 else np.float32(-1.0)
    for K in (3, 10, 20, 30):
        qt = torch.from_numpy(q).cuda()
        kt = torch.from_numpy(k).cuda()
        ix = sp.indexer(qt, kt, None, sp.SCORE_DOT, 1)
        scores = torch.empty(1, 1, Nq, ctx, device="cuda")
        err = torch.empty(1, 1, Nq, device="cuda")
        sp.spattn_index_scores(ix, None, scores, err)
        idx = torch.empty(1, 1, Nq, K, dtype=torch.int32, device="cuda")
        sp.spattn_topk(scores, err, ix, None, K, sp.TOPK_CERTIFIED, idx)
        torch.cuda.synchronize()
        keys = orc.keys_dot(q[0, 0, 0].astype(np.float64), k[0, :, 0].astype(np.float64))
        want = orc.topk(keys, K)
        assert np.array_equal(idx.cpu().numpy()[0, 0, 0], want), K


def test_certified_selection_needs_wide_accumulator():
    """Exact scores a hair off a float32 halfway point: (1 + 2^-12)^2 is the
    midpoint 1 + 2^-11 + 2^-24, and a second product of +-2^-70 decides the
    rounding. The float64 sum rounds (the tracked sum is inexact) and its error
    interval holds the midpoint, so only the wide fixed-point accumulation
    settles these keys: in the row kernels a flagged row is finished by the
    redo kernel with that accumulator."""
    import oracle as orc
    sp = S()
    say("[gpu] certified keys needing the wide accumulator")
    d, ctx, Nq = 8, 96, 4
    a = np.float32(1.0 + 2.0 ** -12)
    t = np.float32(2.0 ** -35)
    q = np.zeros((1, Nq, 1, d), np.float32)
    q[0, :, 0, 0] = a
    q[0, :, 0, 1] = t
    k = np.zeros((1, ctx, 1, d), np.float32)
    for j in range(ctx):
        kind = j % 6
        if kind == 0:
            k[0, j, 0, 0] = np.float32(1.0 + 2.0 ** -10)     # clearly above the midpoint group
        elif kind == 1:
            k[0, j, 0, 0] = np.float32(1.0)                  # clearly below
        else:
            k[0, j, 0, 0] = a
            k[0, j, 0, 1] = [t, -t, np.float32(0.0), t][kind - 2]   # up, down, exactly the midpoint, up
    assert (q.astype(np.float64)[0, 0, 0] @ k.astype(np.float64)[0, 2, 0]) == 1 + 2.0 ** -11 + 2.0 ** -24
    for K in (20, 40, 60):
        qt = torch.from_numpy(q).cuda()
        kt = torch.from_numpy(k).cuda()
        ix = sp.indexer(qt, kt, None, sp.SCORE_DOT, 1)
        scores = torch.empty(1, 1, Nq, ctx, device="cuda")
        err = torch.empty(1, 1, Nq, device="cuda")
        sp.spattn_index_scores(ix, None, scores, err)
        idx = torch.full((1, 1, Nq, K), 7, dtype=torch.int32, device="cuda")
        need = sp.LIB.spattn_topk_workspace(sp.ctypes.byref(sp.tensor(scores)), sp.ctypes.byref(ix), K,
                                            sp.TOPK_CERTIFIED)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
        sp.spattn_topk(scores, err, ix, None, K, sp.TOPK_CERTIFIED, idx, ws=ws)
        torch.cuda.synchronize()
        # the row kernel handed these rows on (one flag word per row at the start of its workspace)
        assert int(ws[: 4 * Nq].view(torch.int32).cpu().count_nonzero()) > 0
        got = idx.cpu().numpy()[0, 0]
        for r in range(Nq):
            p = ctx - Nq + r
            keys = orc.keys_dot(q[0, r, 0].astype(np.float64), k[0, : p + 1, 0].astype(np.float64))
            want = orc.topk(keys, K)
            assert np.array_equal(got[r, : len(want)], want), (K, r)


def _block_select_case(q, k, ctx_len, bs, nb):
    """Run block selection on the GPU and compare every row with the oracle."""
    import oracle as orc
    sp = S()
    B, Hq, Nq, d = q.shape
    Hkv, ctx = k.shape[1], k.shape[2]
    qt, kt = q.cuda(), k.cuda()
    idx = torch.full((B, Hq, Nq, nb), 7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hq, Nq), 7, dtype=torch.int32, device="cuda")
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    sp.spattn_block_select(qt, kt, cl, bs, nb, idx, cnt)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    q64, k64 = q.double().numpy(), k.double().numpy()
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for r in range(Nq):
                p = ctx_len[b] - Nq + r
                want = orc.block_select(q64[b, h, r], k64[b, hk], p, bs, nb) if p >= 0 else np.zeros(0, np.int64)
                assert cnt[b, h, r] == len(want), (b, h, r)
                assert np.array_equal(idx[b, h, r, : len(want)], want), (b, h, r, nb)
                assert np.all(idx[b, h, r, len(want):] == -1)


@pytest.mark.parametrize("case", ["f32_1000_blocks", "bf16_2048_blocks", "bf16_64_blocks_ragged"])
def test_block_select_edges(case):
    """Block routing at every supported block count (per-lane key slots 8/16/32),
    exact ties (duplicate and all-zero blocks), ragged lengths and row tiles."""
    say(f"[gpu] block select {case}")
    g = torch.Generator().manual_seed(11)
    if case == "f32_1000_blocks":
        B, Hq, Hkv, Nq, d, ctx, bs = 2, 2, 1, 24, 64, 2000, 2
        q = torch.randn(B, Hq, Nq, d, generator=g)
        k = torch.randn(B, Hkv, ctx, d, generator=g)
        for src, dst in ((5, 9), (5, 700), (11, 12)):            # tied keys: identical blocks
            k[:, :, dst * bs:(dst + 1) * bs] = k[:, :, src * bs:(src + 1) * bs]
        k[1, :, 100 * bs:400 * bs] = 0.0                          # a run of exact-zero keys
        for nb in (1, 37, 999):
            _block_select_case(q, k, [2000, 1337], bs, nb)
    elif case == "bf16_2048_blocks":
        B, Hq, Hkv, Nq, d, ctx, bs = 1, 2, 2, 9, 128, 2048, 1
        q = torch.randn(B, Hq, Nq, d, generator=g).bfloat16()
        k = torch.randn(B, Hkv, ctx, d, generator=g).bfloat16()
        k[0, 1] = 0.0                                              # head 1: every key ties at 0
        k[0, 0, 1000:1010] = k[0, 0, 3]
        for nb in (100, 2047):
            _block_select_case(q, k, [2048], bs, nb)
    else:
        B, Hq, Hkv, Nq, d, ctx, bs = 2, 4, 2, 70, 128, 4096, 64
        q = torch.randn(B, Hq, Nq, d, generator=g).bfloat16()
        k = torch.randn(B, Hkv, ctx, d, generator=g).bfloat16()
        k[:, :, 64 * 10:64 * 11] += 1.5                           # a strongly preferred block
        for nb in (3, 16, 63):
            _block_select_case(q, k, [4096, 1000], bs, nb)


# ---------------------------------------------------------------- full-size workloads
def test_decode_full_every_row():
    wl = gen.WORKLOADS["dsa_decode"]
    say("[gpu] generating dsa_decode inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


def _sample_rows(wl, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(min(8, wl.Nq)))
    rows |= {wl.Nq - 1, wl.Nq - 2}
    rows |= set(int(x) for x in rng.integers(0, wl.Nq, size=n))
    return [(0, r) for r in sorted(rows)]


@pytest.mark.parametrize("name,n", [("window_global", 48), ("block_sparse", 24), ("dsa_prefill", 24),
                                    ("window_stride", 48), ("nsa_blocks", 16), ("msa_prefill", 16)])
def test_full_size_sampled_rows(name, n):
    wl = gen.WORKLOADS[name]
    say(f"[gpu] generating {name} inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _sample_rows(wl, n, 11)
    if name == "dsa_prefill":
        rows += [(0, int(i)) for i in inp["needles"][:8, 1]]
    res = oracle_rows(wl, inp, rows)
    if hp.idx is not None:
        check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)
    if name == "dsa_prefill":
        idx = hp.idx.cpu().numpy()
        for (b, i, j) in inp["needles"]:
            assert j in idx[b, 0, i]


# ---------------------------------------------------------------- fused indexer + top-K
def run_fused(wl, inp):
    from fine_grained_top_amd.hotpath import HotPath
    say(f"[gpu] fused {wl.name}: B={wl.B} N={wl.N} Nq={wl.Nq}")
    hp = HotPath(wl, inp, fused=True)
    hp.step()
    torch.cuda.synchronize()
    return hp


@pytest.mark.parametrize("name", ["dsa_decode_small", "dsa_decode", "dsa_prefill_small"])
def test_fused_index_topk(name):
    wl = gen.WORKLOADS[name]
    inp = gen.generate(wl)
    hp = run_fused(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


def test_fused_falls_back_when_the_sample_misleads():
    """Keys inside the pilot's sample runs are made to score zero, so the
    sampled threshold is useless; the fused call must still be exact."""
    wl = dataclasses.replace(gen.WORKLOADS["dsa_decode_small"], B=2, N=40000, len_range=(36000, 40000), topk=512)
    inp = gen.generate(wl)
    codes = inp["k_idx"]
    pos = np.arange(wl.N)
    inside = (pos % 2048) < 64
    codes[:, inside, 0, :] = 0                    # +0 keys: every score in the sample is 0
    hp = run_fused(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)


@pytest.mark.parametrize("kfmt,layout", [("fp8", "one_run"), ("bf16", "one_run"), ("fp8", "short_runs")])
def test_fused_decode_clustered_extreme_keys(kfmt, layout):
    """Decode rows whose survivors crowd into a few 512-key chunks (more than
    a thread of the final selection loads in its first round) and whose
    largest scores are far above the rest (so the score range is split twice
    by the selection histogram): runs of large indexer keys, distinct by
    position, are planted in every request; fp8 and bf16 indexer keys. One
    run of 300 keys puts more extra slots in one wave of the final selection
    than its LDS region holds (they are read from global memory in every
    pass); three runs of 50 keys in chunks of different waves fit the
    regions."""
    wl = dataclasses.replace(gen.WORKLOADS["dsa_decode_small"], B=2, N=40000, len_range=(36000, 40000), topk=512,
                             idx_k_dtype=kfmt)
    inp = gen.generate(wl)
    codes = inp["k_idx"]
    if layout == "one_run":
        run = np.arange(5000, 5300)
    else:
        run = np.concatenate([np.arange(1030, 1080), np.arange(9230, 9280), np.arange(20030, 20080)])
    if kfmt == "fp8":
        codes[:, run, 0, :] = (0x68 + (run % 8)).astype(codes.dtype)[:, None]      # 64 .. 120
    else:
        codes[:, run, 0, :] = (0x4200 + (run % 128)).astype(codes.dtype)[:, None]    # 32 .. 63.75
    hp = run_fused(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


# ---------------------------------------------------------------- modes agree
def test_dense_mode_small():
    wl = gen.WORKLOADS["dense_small"]
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_out(hp, res, rows, 2e-3)


def test_index_mode_equals_window_global_mode():
    """Index mode fed the expanded window/global lists reproduces the
    window/global mode ('A Guide to Sparse Attention', index-based vs fixed
    patterns): the two kernels agree to float32 rounding."""
    import oracle as orc
    sp = S()
    wl = gen.WORKLOADS["window_global_small"]
    inp = gen.generate(wl)
    hp = run(wl, inp)                                   # window/global mode
    o_pattern = hp.o.clone()
    width = wl.window + wl.n_global
    lists = np.full((wl.B, 1, wl.Nq, width), -1, np.int32)
    for r in range(wl.Nq):
        p = wl.N - wl.Nq + r
        sset = sorted(set(range(max(0, p - wl.window + 1), p + 1)) | set(range(min(wl.n_global, p + 1))))
        lists[0, 0, r, : len(sset)] = sset
    idx = torch.from_numpy(lists).cuda()
    o = torch.empty_like(hp.o)
    sp.spattn_sparse_attn_fwd(hp.q, hp.k, hp.v, hp.ctx_len, 0.0, sp.selection(sp.SEL_INDEX, idx), o)
    torch.cuda.synchronize()
    diff = float((o - o_pattern).abs().max())
    say(f"  index vs pattern max diff {diff:.3e}")
    assert diff <= 2e-3


@pytest.mark.parametrize("bs", [64, 32, 128])
def test_blocks_attention_edge_lists(bs):
    """BLOCKS mode with hand-made lists: repeated blocks, padding, blocks after
    the row, blocks inside the window, rows whose blocks all lie in the window,
    ragged lengths, several requests and heads; every row against the oracle's
    masked attention over the union of the blocks and the window."""
    import oracle as orc
    sp = S()
    say(f"[gpu] blocks attention edge lists bs={bs}")
    g = torch.Generator().manual_seed(21)
    B, Hq, Hkv, Nq, d, ctx, nb, w = 2, 4, 2, 300, 128, 1200, 6, 100
    q = torch.randn(B, Hq, Nq, d, generator=g).bfloat16()
    k = torch.randn(B, Hkv, ctx, d, generator=g).bfloat16()
    v = torch.randn(B, Hkv, ctx, d, generator=g).bfloat16()
    ctx_len = [1200, 777]
    nbk = ctx // bs
    rng = np.random.default_rng(22)
    blk = rng.integers(-1, nbk, size=(B, Hq, Nq, nb)).astype(np.int32)
    blk[..., 1] = blk[..., 0]                                  # a repeated block
    blk[0, 0, :, :] = nbk - 1                                   # after most rows' positions
    blk[1, 1, ::3, 2:] = -1                                     # padding
    for r in range(Nq):                                         # blocks inside the window
        p = ctx_len[1] - Nq + r
        blk[1, 2, r, 3] = max(0, p // bs)
    qt, kt, vt = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty(B, Hq, Nq, d, device="cuda")
    lse = torch.empty(B, Hq, Nq, device="cuda")
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    sel = sp.selection(sp.SEL_BLOCKS, torch.from_numpy(blk).cuda(), window=w, block_size=bs)
    sp.spattn_sparse_attn_fwd(qt, kt, vt, cl, 0.0, sel, o, lse)
    torch.cuda.synchronize()
    O, LS = o.cpu().numpy(), lse.cpu().numpy()
    q64, k64, v64 = q.double().numpy(), k.double().numpy(), v.double().numpy()
    worst = 0.0
    for b in range(B):
        L = ctx_len[b]
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            for r in range(Nq):
                p = L - Nq + r
                blocks = [int(x) for x in blk[b, h, r] if 0 <= x < nbk]
                S_ = orc.blocks_set(blocks, p, bs, w)
                Oo, Lo = orc.masked_attention(q64[b, h, r][None], k64[b, kvh, : p + 1], v64[b, kvh, : p + 1], S_,
                                              1.0 / math.sqrt(d))
                worst = max(worst, float(np.abs(O[b, h, r] - Oo[0]).max()), abs(float(LS[b, h, r] - Lo[0])))
    say(f"  max |O - O_oracle|, |LSE - LSE_oracle| = {worst:.3e}")
    assert worst <= 2e-3


# ---------------------------------------------------------------- page-granular selection, paged KV
def _page_select_on(sc, P, top, n_local, ctx_len):
    sp = S()
    B, G, nq, ctx = sc.shape
    idx = torch.full((B, G, nq, top + n_local), 7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, G, nq), 7, dtype=torch.int32, device="cuda")
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    sp.spattn_page_select(sc, None, None, cl, P, top, n_local, 0, idx, cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def _check_pages(idx, cnt, keys_of, ctx_len, Nq, P, top, n_local):
    import oracle as orc
    B, G = idx.shape[:2]
    for b in range(B):
        for g in range(G):
            for r in range(Nq):
                p = ctx_len[b] - Nq + r
                want = orc.page_select(keys_of(b, g, r, p), p, P, top, n_local)
                assert cnt[b, g, r] == len(want), (P, top, n_local, b, g, r)
                assert np.array_equal(idx[b, g, r, : len(want)], want), (P, top, n_local, b, g, r)
                assert np.all(idx[b, g, r, len(want):] == -1)


@pytest.mark.parametrize("ctx", [3000, 3001])
def test_page_select_ties_and_edges(ctx):
    """Uncertified page selection on integer scores (many tied page keys), +-0,
    a row of equal scores, ragged lengths, page sizes from 1 to 512, rows that
    are and are not 16-byte aligned (odd row length), and top_pages from 0 to
    more than the candidate pages."""
    say(f"[gpu] page select ties/edges ctx={ctx}")
    rng = np.random.default_rng(31)
    B, G, Nq = 2, 2, 12
    sc = rng.integers(-6, 7, size=(B, G, Nq, ctx)).astype(np.float32)
    sc[0, 0, 3] = 1.0
    sc[1, 1, :, ::3] = -0.0
    sc[1, 1, :, 1::3] = 0.0
    ctx_len = [ctx, 1777]
    dev = torch.from_numpy(sc).cuda()
    for P, top, n_local in [(1, 40, 0), (1, 5, 3), (4, 7, 1), (16, 5, 2), (16, 0, 3), (64, 6, 2), (64, 1, 0),
                            (128, 3, 1), (512, 1, 1), (64, 1000, 2), (4096, 1, 0)]:
        idx, cnt = _page_select_on(dev, P, top, n_local, ctx_len)
        _check_pages(idx, cnt, lambda b, g, r, p: sc[b, g, r, : p + 1], ctx_len, Nq, P, top, n_local)


def _dot_page_case(q, k, P, top, n_local, Nq):
    """Certified page selection from indexer scores (DOT, f32) against the
    oracle's exact keys."""
    import oracle as orc
    sp = S()
    ctx = k.shape[1]
    qt = torch.from_numpy(q).cuda()
    kt = torch.from_numpy(k).cuda()
    ix = sp.indexer(qt, kt, None, sp.SCORE_DOT, 1)
    scores = torch.empty(1, 1, Nq, ctx, device="cuda")
    err = torch.empty(1, 1, Nq, device="cuda")
    sp.spattn_index_scores(ix, None, scores, err)
    idx = torch.full((1, 1, Nq, top + n_local), 7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, 1, Nq), 7, dtype=torch.int32, device="cuda")
    sp.spattn_page_select(scores, err, ix, None, P, top, n_local, sp.TOPK_CERTIFIED, idx, cnt)
    torch.cuda.synchronize()
    keys = lambda b, g, r, p: orc.keys_dot(q[0, r, 0].astype(np.float64), k[0, : p + 1, 0].astype(np.float64))
    _check_pages(idx.cpu().numpy(), cnt.cpu().numpy(), keys, [ctx], Nq, P, top, n_local)


def test_page_select_certified_near_ties():
    """Token scores at and a hair off float32 halfway points (the second
    product of +-2^-70 needs the wide fixed-point accumulation): page keys tie
    in float32 and only the exact keys order the pages."""
    say("[gpu] certified page select near ties")
    d, ctx, Nq = 8, 96, 4
    a = np.float32(1.0 + 2.0 ** -12)
    t = np.float32(2.0 ** -35)
    q = np.zeros((1, Nq, 1, d), np.float32)
    q[0, :, 0, 0] = a
    q[0, :, 0, 1] = t
    k = np.zeros((1, ctx, 1, d), np.float32)
    for j in range(ctx):
        kind = j % 6
        if kind == 0:
            k[0, j, 0, 0] = np.float32(1.0 + 2.0 ** -10)
        elif kind == 1:
            k[0, j, 0, 0] = np.float32(1.0)
        else:
            k[0, j, 0, 0] = a
            k[0, j, 0, 1] = [t, -t, np.float32(0.0), t][kind - 2]
    for P, top, n_local in [(1, 20, 0), (1, 40, 2), (2, 12, 1), (4, 5, 0), (8, 3, 1)]:
        _dot_page_case(q, k, P, top, n_local, Nq)
    # pages whose best tokens sit at rounding midpoints of the plain dot product
    q2 = np.zeros((1, 2, 1, d), np.float32)
    q2[0, :, 0, :2] = 1.0
    k2 = np.zeros((1, 64, 1, d), np.float32)
    k2[0, :, 0, 0] = 1.0
    tiny = np.float32(2.0 ** -24)
    pattern = [tiny, tiny + np.float32(2.0 ** -40), 0.0, 3 * tiny]
    for j in range(64):
        k2[0, j, 0, 1] = pattern[j % 4] if j % 5 else np.float32(-1.0)
    for P, top, n_local in [(1, 10, 0), (2, 6, 1), (4, 3, 2)]:
        _dot_page_case(q2, k2, P, top, n_local, 2)


def test_paged_decode_full_every_row():
    wl = gen.WORKLOADS["dsa_paged_decode"]
    say("[gpu] generating dsa_paged_decode inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


def _pool(x, table, P):
    """[B, Hkv, ctx, d] -> a page pool [B * npr, Hkv, P, d] laid out by the page table."""
    B, Hkv, ctx, d = x.shape
    npr = table.shape[1]
    pad = npr * P - ctx
    xp = torch.cat([x, torch.zeros(B, Hkv, pad, d, dtype=x.dtype)], dim=2) if pad else x
    logical = xp.reshape(B, Hkv, npr, P, d).permute(0, 2, 1, 3, 4).reshape(B * npr, Hkv, P, d)
    pool = torch.empty_like(logical)
    pool[torch.from_numpy(table.reshape(-1)).long()] = logical
    return pool.contiguous()


@pytest.mark.parametrize("dtype,d,Nq", [("bf16", 128, 1), ("bf16", 128, 40), ("f32", 64, 40)])
def test_paged_storage_matches_contiguous(dtype, d, Nq):
    """Attention over a paged pool reads the same keys as over the contiguous
    cache: with the same kernel the outputs agree bit for bit, for index lists
    and for page lists; page lists also agree bit for bit with the index lists
    they expand to, and every row matches the oracle."""
    import oracle as orc
    sp = S()
    say(f"[gpu] paged vs contiguous {dtype} d={d} Nq={Nq}")
    g = torch.Generator().manual_seed(41)
    B, Hq, Hkv, ctx, P, npg = 3, 8, 2, 1000, 16, 9
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(B, Hq, Nq, d, generator=g).to(tdt)
    k = torch.randn(B, Hkv, ctx, d, generator=g).to(tdt)
    v = torch.randn(B, Hkv, ctx, d, generator=g).to(tdt)
    ctx_len = [1000, 777, 513]
    npr = (ctx + P - 1) // P
    table = np.random.default_rng(42).permutation(B * npr).astype(np.int32).reshape(B, npr)
    kp, vp = _pool(k, table, P), _pool(v, table, P)
    rng = np.random.default_rng(43)
    plist = np.full((B, Hkv, Nq, npg), -1, np.int32)
    tlist = np.full((B, Hkv, Nq, npg * P), -1, np.int32)
    for b in range(B):
        for gg in range(Hkv):
            for r in range(Nq):
                p = ctx_len[b] - Nq + r
                last = p // P
                n = int(rng.integers(1, npg + 1))
                pages = np.sort(rng.choice(np.arange(last + 2), size=min(n, last + 2), replace=False))
                plist[b, gg, r, : len(pages)] = pages             # may include the page after p
                toks = np.concatenate([np.arange(P * x, P * x + P) for x in pages])
                tlist[b, gg, r, : len(toks)] = toks
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kpd, vpd = kp.cuda(), vp.cuda()
    tab = torch.from_numpy(table).cuda()
    pages = sp.kv_pages(tab, P)
    pld, tld = torch.from_numpy(plist).cuda(), torch.from_numpy(tlist).cuda()
    outs = {}
    for name, sel in [("pages", sp.selection(sp.SEL_PAGES, pld, block_size=P)),
                      ("index", sp.selection(sp.SEL_INDEX, tld))]:
        for paged in (False, True):
            o = torch.empty(B, Hq, Nq, d, device="cuda")
            lse = torch.empty(B, Hq, Nq, device="cuda")
            if paged:
                sp.spattn_sparse_attn_fwd_paged(qd, kpd, vpd, pages, cl, 0.0, sel, o, lse)
            else:
                sp.spattn_sparse_attn_fwd(qd, kd, vd, cl, 0.0, sel, o, lse)
            torch.cuda.synchronize()
            outs[(name, paged)] = (o.cpu(), lse.cpu())
    ref_o, ref_l = outs[("index", False)]
    for key, (o, l) in outs.items():
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), key
    q64, k64, v64 = q.double().numpy(), k.double().numpy(), v.double().numpy()
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            for r in range(Nq):
                p = ctx_len[b] - Nq + r
                S_ = orc.pages_set([x for x in plist[b, kvh, r] if x >= 0], p, P)
                if len(S_) == 0:                                  # only the page after p was listed
                    assert torch.all(ref_o[b, h, r] == 0) and float(ref_l[b, h, r]) == -math.inf
                    continue
                o, l = orc.masked_attention(q64[b, h, r][None], k64[b, kvh, : p + 1], v64[b, kvh, : p + 1], S_,
                                            1.0 / math.sqrt(d))
                worst = max(worst, float(np.abs(ref_o[b, h, r].double().numpy() - o[0]).max()),
                            abs(float(ref_l[b, h, r]) - float(l[0])))
    tol = 1e-5 if dtype == "f32" else 2e-3
    say(f"  max diff vs oracle {worst:.3e} (tol {tol})")
    assert worst <= tol


@pytest.mark.parametrize("name,P,top", [("dsa_paged_decode_small", 64, 6), ("dsa_paged_decode_small", 32, 9),
                                        ("dsa_paged_decode_small", 512, 1), ("dsa_paged_decode_small", 16, 20),
                                        ("dsa_paged_prefill_small", 16, 5), ("dsa_paged_prefill_small", 128, 1),
                                        ("dsa_paged_decode", 64, 30)])
def test_fused_page_select(name, P, top):
    """Page selection from the indexer inputs in one call: the page keys come
    from the indexer's epilogue (pages of 32..512 keys on its MFMA path) or
    from the separate page-key pass; page lists equal the oracle's and the
    two-call path's bit for bit, and the attention over them matches."""
    wl = dataclasses.replace(gen.WORKLOADS[name], page_size=P, top_pages=top)
    inp = gen.generate(wl)
    hp = run_fused(wl, inp)
    rows = _all_rows(wl, inp) if wl.Nq == 1 else [(0, r) for r in range(0, wl.Nq, 7)] + [(0, wl.Nq - 1)]
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)
    fused_idx = hp.idx.clone()
    hp.index_scores()
    hp.page_select()
    torch.cuda.synchronize()
    assert torch.equal(hp.idx, fused_idx)


@pytest.mark.parametrize("stride,g,w,dtype", [(8, 0, 65, "bf16"), (64, 5, 100, "bf16"), (100, 3, 40, "bf16"),
                                              (1, 0, 10, "bf16"), (7, 2, 30, "f32")])
def test_window_stride_modes_agree(stride, g, w, dtype):
    """The strided window/global pattern against index lists that spell out
    the same visible sets (the tiled kernel, or the generic one for f32,
    against the gather kernel), and every row against the oracle."""
    import oracle as orc
    sp = S()
    say(f"[gpu] window+stride s={stride} g={g} w={w} {dtype}")
    g_ = torch.Generator().manual_seed(51)
    B, H, Nq, ctx, d = 2, 2, 300, 700, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(B, H, Nq, d, generator=g_).to(tdt)
    k = torch.randn(B, H, ctx, d, generator=g_).to(tdt)
    v = torch.randn(B, H, ctx, d, generator=g_).to(tdt)
    ctx_len = [700, 455]
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    o_pat = torch.empty(B, H, Nq, d, device="cuda")
    l_pat = torch.empty(B, H, Nq, device="cuda")
    sp.spattn_sparse_attn_fwd(qd, kd, vd, cl, 0.0, sp.selection(sp.SEL_WINDOW_GLOBAL, window=w, n_global=g,
                                                                 stride=stride), o_pat, l_pat)
    sets = {}
    width = 0
    for b in range(B):
        for r in range(Nq):
            p = ctx_len[b] - Nq + r
            sets[(b, r)] = orc.window_global_set(p, w, g, stride)
            width = max(width, len(sets[(b, r)]))
    lists = np.full((B, 1, Nq, width), -1, np.int32)
    for (b, r), S_ in sets.items():
        lists[b, 0, r, : len(S_)] = S_
    ld = torch.from_numpy(lists).cuda()
    o_idx = torch.empty_like(o_pat)
    sp.spattn_sparse_attn_fwd(qd, kd, vd, cl, 0.0, sp.selection(sp.SEL_INDEX, ld), o_idx)
    torch.cuda.synchronize()
    diff = float((o_idx - o_pat).abs().max())
    q64, k64, v64 = q.double().numpy(), k.double().numpy(), v.double().numpy()
    O, LSE = o_pat.cpu().numpy(), l_pat.cpu().numpy()
    worst = 0.0
    for (b, r), S_ in sets.items():
        p = ctx_len[b] - Nq + r
        for h in range(H):
            o, l = orc.masked_attention(q64[b, h, r][None], k64[b, h, : p + 1], v64[b, h, : p + 1], S_,
                                        1.0 / math.sqrt(d))
            worst = max(worst, float(np.abs(O[b, h, r] - o[0]).max()), abs(float(LSE[b, h, r]) - float(l[0])))
    tol = 1e-5 if dtype == "f32" else 2e-3
    say(f"  pattern vs index lists {diff:.3e}; pattern vs oracle {worst:.3e} (tol {tol})")
    assert worst <= tol and diff <= tol


def test_nsa_branches_one_at_a_time():
    """One-hot gates return one branch: the window branch equals the window
    mode, the selection branch equals the blocks mode without a window (bit
    for bit: the same kernels), the compression branch matches the oracle's
    attention over the block means rounded to bf16."""
    import oracle as orc
    sp = S()
    wl = gen.WORKLOADS["nsa_blocks_small"]
    inp = gen.generate(wl)
    hp = run(wl, inp)
    B, H, Nq, d = wl.B, wl.Hq, wl.Nq, wl.d
    outs = []
    for g in ((1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0)):
        gates = torch.tensor(g, device="cuda").view(1, 1, 1, 3).expand(B, H, Nq, 3).contiguous()
        o = torch.empty(B, H, Nq, d, device="cuda")
        sp.spattn_nsa_fwd(hp.q, hp.k, hp.v, hp.ctx_len, 0.0, wl.block_size, hp.idx, wl.window, gates, o)
        outs.append(o)
    o_blk = torch.empty_like(outs[0])
    sp.spattn_sparse_attn_fwd(hp.q, hp.k, hp.v, hp.ctx_len, 0.0,
                              sp.selection(sp.SEL_BLOCKS, hp.idx, window=0, block_size=wl.block_size), o_blk)
    o_win = torch.empty_like(outs[0])
    sp.spattn_sparse_attn_fwd(hp.q, hp.k, hp.v, hp.ctx_len, 0.0,
                              sp.selection(sp.SEL_WINDOW_GLOBAL, window=wl.window), o_win)
    torch.cuda.synchronize()
    assert torch.equal(outs[1], o_blk) and torch.equal(outs[2], o_win)
    q64 = orc.decode(inp["q"][0], "bf16")
    k64 = orc.decode(inp["k"][0], "bf16")
    v64 = orc.decode(inp["v"][0], "bf16")
    O = outs[0].cpu().numpy()
    worst = 0.0
    qpk = H // wl.Hkv
    nb = Nq // wl.block_size
    pooled = [(orc.pooled_blocks(k64[x], wl.block_size, nb), orc.pooled_blocks(v64[x], wl.block_size, nb))
              for x in range(wl.Hkv)]
    for r in list(range(0, 70)) + list(range(70, Nq, 37)):
        for h in range(H):
            got = O[0, h, r]
            want = orc.nsa_attention(q64[h, r], k64[h // qpk], v64[h // qpk], r, wl.block_size, [], wl.window,
                                     np.array([1.0, 0.0, 0.0]), 1 / math.sqrt(d),
                                     pooled=pooled[h // qpk])
            worst = max(worst, float(np.abs(got - want).max()))
    say(f"  compression branch vs oracle {worst:.3e}")
    assert worst <= 2e-3


def test_two_level_decode_full_every_row():
    wl = gen.WORKLOADS["dsa_two_level_decode"]
    say("[gpu] generating dsa_two_level_decode inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


@pytest.mark.parametrize("bs,nb,K", [(4, 3, 10), (4, 30, 50), (8, 2, 7), (1, 12, 12), (16, 1, 40)])
def test_two_level_certified_near_ties(bs, nb, K):
    """Token and block keys at and a hair off float32 halfway points (the
    second product of +-2^-70 needs the wide accumulator), f32 DOT indexer:
    both picks against the oracle's exact keys; also top_blocks beyond the
    blocks and K beyond the candidates."""
    import oracle as orc
    sp = S()
    say(f"[gpu] two-level near ties bs={bs} nb={nb} K={K}")
    d, ctx, Nq = 8, 96, 4
    a = np.float32(1.0 + 2.0 ** -12)
    t = np.float32(2.0 ** -35)
    q = np.zeros((1, Nq, 1, d), np.float32)
    q[0, :, 0, 0] = a
    q[0, :, 0, 1] = t
    k = np.zeros((1, ctx, 1, d), np.float32)
    for j in range(ctx):
        kind = (j * 7) % 6
        if kind == 0:
            k[0, j, 0, 0] = np.float32(1.0 + 2.0 ** -10)
        elif kind == 1:
            k[0, j, 0, 0] = np.float32(1.0)
        else:
            k[0, j, 0, 0] = a
            k[0, j, 0, 1] = [t, -t, np.float32(0.0), t][kind - 2]
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda()
    ix = sp.indexer(qt, kt, None, sp.SCORE_DOT, 1)
    kb = torch.empty(1, ctx // bs, 1, d, device="cuda")
    sp.spattn_pool_index_keys(ix, None, bs, kb)
    idx = torch.full((1, 1, Nq, K), 7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, 1, Nq), 7, dtype=torch.int32, device="cuda")
    sp.spattn_topk_two_level(ix, kb, None, bs, nb, K, idx, cnt)
    torch.cuda.synchronize()
    got, gc = idx.cpu().numpy()[0, 0], cnt.cpu().numpy()[0, 0]
    k64 = k[0, :, 0].astype(np.float64)
    for r in range(Nq):
        p = ctx - Nq + r
        q64 = q[0, r, 0].astype(np.float64)
        tk = orc.keys_dot(q64, k64[: p + 1])
        nbe = (p + 1) // bs
        bk = orc.keys_dot(q64, orc.pooled_blocks(k64, bs, nbe, "f32"))
        want = orc.two_level_select(bk, tk, p, bs, nb, K)
        assert gc[r] == len(want), (r, gc[r], len(want))
        assert np.array_equal(got[r, : len(want)], want), r
        assert np.all(got[r, len(want):] == -1)



# ---------------------------------------------------------------- backward
def _grads_oracle(q, k, v, dO, sets, ctx_len, Nq, scale):
    """dq, dk, dv by the oracle: per (request, head, row) gradients of the
    masked attention, the key gradients summed over rows and heads."""
    import oracle as orc
    B, Hq, _, d = q.shape
    Hkv, ctx = k.shape[1], k.shape[2]
    dq = np.zeros((B, Hq, Nq, d))
    dk = np.zeros((B, Hkv, ctx, d))
    dv = np.zeros((B, Hkv, ctx, d))
    for b in range(B):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            for r in range(Nq):
                p = ctx_len[b] - Nq + r
                S_ = sets(b, h, r, p)
                gq, gk, gv = orc.masked_attention_grads(q[b, h, r][None], k[b, kvh, : p + 1], v[b, kvh, : p + 1],
                                                        S_, scale, dO[b, h, r][None])
                dq[b, h, r] = gq[0]
                dk[b, kvh, : p + 1] += gk
                dv[b, kvh, : p + 1] += gv
    return dq, dk, dv


@pytest.mark.parametrize("mode,dtype", [("window", "bf16"), ("window_wide", "bf16"), ("window_long", "bf16"), ("stride", "f32"),
                                        ("index", "bf16"), ("blocks", "bf16"), ("dense", "f32"), ("dense", "bf16")])
def test_attention_backward(mode, dtype):
    """dq, dk, dv over every selection mode, GQA, ragged lengths, against the
    oracle's gradients (float32 accumulation with float atomics). The bf16
    dense and window cases run the tiled kernel (query tiles of 64 rows, one
    full and one ragged, over ragged key tiles), the others the per-row one.
    window_long has room for 320 keys and requests of 300 and 130: a band key
    tile that no query tile sees and key tiles past a request's length, whose
    gradient rows are written as zeros by the slot reduce."""
    import oracle as orc
    sp = S()
    say(f"[gpu] backward {mode} {dtype}")
    g_ = torch.Generator().manual_seed(61)
    B, Hq, Hkv, Nq, ctx = 2, 4, 2, 96, (320 if mode == "window_long" else 160)
    d = 128 if dtype == "bf16" else 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(B, Hq, Nq, d, generator=g_).to(tdt)
    k = torch.randn(B, Hkv, ctx, d, generator=g_).to(tdt)
    v = torch.randn(B, Hkv, ctx, d, generator=g_).to(tdt)
    dO = torch.randn(B, Hq, Nq, d, generator=g_)
    ctx_len = [300, 130] if mode == "window_long" else [160, 130]
    rng = np.random.default_rng(62)
    keep = []
    if mode in ("window", "window_wide", "window_long", "stride"):
        w, gl, st = (70, 17, 0) if mode == "window_wide" else (20, 3, (7 if mode == "stride" else 0))
        sel = sp.selection(sp.SEL_WINDOW_GLOBAL, window=w, n_global=gl, stride=st)
        sets = lambda b, h, r, p: orc.window_global_set(p, w, gl, st)
    elif mode == "index":
        lists = np.full((B, Hkv, Nq, 24), -1, np.int32)
        for b in range(B):
            for g in range(Hkv):
                for r in range(Nq):
                    p = ctx_len[b] - Nq + r
                    s_ = np.sort(rng.choice(p + 1, size=min(24, p + 1), replace=False))
                    lists[b, g, r, : len(s_)] = s_
        ld = torch.from_numpy(lists).cuda()
        keep.append(ld)
        sel = sp.selection(sp.SEL_INDEX, ld)
        sets = lambda b, h, r, p: lists[b, h // (Hq // Hkv), r][lists[b, h // (Hq // Hkv), r] >= 0]
    elif mode == "blocks":
        bs, nb, w = 16, 3, 10
        blk = np.full((B, Hq, Nq, nb), -1, np.int32)
        for b in range(B):
            for h in range(Hq):
                for r in range(Nq):
                    p = ctx_len[b] - Nq + r
                    ne = (p + 1) // bs
                    c = np.sort(rng.choice(ne, size=min(nb, ne), replace=False)) if ne else []
                    blk[b, h, r, : len(c)] = c
        bd = torch.from_numpy(blk).cuda()
        keep.append(bd)
        sel = sp.selection(sp.SEL_BLOCKS, bd, window=w, block_size=bs)
        sets = lambda b, h, r, p: orc.blocks_set([x for x in blk[b, h, r] if x >= 0], p, bs, w)
    else:
        sel = sp.selection(sp.SEL_DENSE)
        sets = lambda b, h, r, p: np.arange(p + 1)
    qd, kd, vd, dOd = q.cuda(), k.cuda(), v.cuda(), dO.cuda()
    cl = torch.tensor(ctx_len, dtype=torch.int32, device="cuda")
    o = torch.empty(B, Hq, Nq, d, device="cuda")
    lse = torch.empty(B, Hq, Nq, device="cuda")
    sp.spattn_sparse_attn_fwd(qd, kd, vd, cl, 0.0, sel, o, lse)
    dq = torch.empty(B, Hq, Nq, d, device="cuda")
    dk = torch.full((B, Hkv, ctx, d), float("nan"), device="cuda")
    dv = torch.full((B, Hkv, ctx, d), float("nan"), device="cuda")
    # workspace filled with NaN: a slot the reduce reads but nobody wrote would show
    nws = sp.spattn_sparse_attn_bwd_workspace(qd, kd, sel)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda") if nws else None
    sp.spattn_sparse_attn_bwd(qd, kd, vd, cl, 0.0, sel, o, lse, dOd, dq, dk, dv, ws)
    torch.cuda.synchronize()
    rq, rk, rv = _grads_oracle(q.double().numpy(), k.double().numpy(), v.double().numpy(), dO.double().numpy(),
                               sets, ctx_len, Nq, 1.0 / math.sqrt(d))
    errs = [float(np.abs(got.cpu().numpy() - ref).max()) / max(1.0, float(np.abs(ref).max()))
            for got, ref in ((dq, rq), (dk, rk), (dv, rv))]
    say(f"  relative max errors dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    assert max(errs) <= 1e-4


# ---------------------------------------------------------------- Quest page selection
def _quest_case(dtype, d, tails):
    """A paged cache whose page keys sit on float32 rounding midpoints and tie
    often: query (1, 1, 0, ...), every key's channel 0 is 1 and channel 1 one
    of `tails`, so a page's bound is 1 + its largest tail (one head)."""
    B, Hkv, P, npg = 2, 2, 4, 40
    ctx = P * npg
    rng = np.random.default_rng(71)
    K = np.zeros((B, Hkv, ctx, d), np.float64)
    K[..., 0] = 1.0
    K[..., 1] = np.array(tails)[rng.integers(0, len(tails), size=(B, Hkv, ctx))]
    K[..., 2:] = rng.integers(-2, 3, size=(B, Hkv, ctx, d - 2))
    q = np.zeros((B, Hkv, 1, d), np.float64)
    q[..., 0] = 1.0
    q[..., 1] = 1.0
    return K, q, P, npg


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_quest_bounds_and_ties(dtype, d):
    """Per-page bounds equal the exact channel minima and maxima; page lists
    equal the oracle's where many bounds tie and sit on float32 midpoints (the
    exact-sum path), with a partial last page and ragged lengths."""
    import oracle as orc
    sp = S()
    say(f"[gpu] quest bounds and ties {dtype} d={d}")
    tails = [0.0, 2.0 ** -24, 3 * 2.0 ** -24, -(2.0 ** -25), -3 * 2.0 ** -25, 2.0 ** -20]
    K, q, P, npg = _quest_case(dtype, d, tails)
    B, Hkv, ctx, _ = K.shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # pool: logical page (b, pg) at slot perm[b * npg + pg]
    perm = np.random.default_rng(72).permutation(B * npg)
    pool = np.zeros((B * npg, Hkv, P, d))
    table = np.zeros((B, npg), np.int32)
    for b in range(B):
        for pg in range(npg):
            pool[perm[b * npg + pg]] = K[b, :, pg * P:(pg + 1) * P]
            table[b, pg] = perm[b * npg + pg]
    kp = torch.from_numpy(pool).to(tdt).cuda()
    tab = torch.from_numpy(table).cuda()
    pages = sp.kv_pages(tab, P)
    lens = [ctx, ctx - 7]
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bnd = torch.full((B, npg, Hkv, 2 * d), float("nan"), dtype=tdt, device="cuda")
    sp.spattn_quest_page_bounds(kp, pages, cl, bnd)
    qd = torch.from_numpy(q).to(tdt).cuda()
    for top, loc in ((5, 1), (12, 2), (40, 1)):
        io = torch.empty(B, Hkv, 1, top + loc, dtype=torch.int32, device="cuda")
        cnt = torch.empty(B, Hkv, 1, dtype=torch.int32, device="cuda")
        sp.spattn_quest_select(qd, bnd, cl, P, top, loc, io, cnt)
        torch.cuda.synchronize()
        got, gc = io.cpu().numpy(), cnt.cpu().numpy()
        for b in range(B):
            p = lens[b] - 1
            for h in range(Hkv):
                want = orc.quest_select(q[b, h], K[b, h], p, P, top, loc)
                assert gc[b, h, 0] == len(want) and np.array_equal(got[b, h, 0, :len(want)], want), (b, h, top)
                assert np.all(got[b, h, 0, len(want):] == -1)
    bn = bnd.float().cpu().numpy()
    for b in range(B):
        for pg in range(lens[b] // P):
            rows = K[b, :, pg * P:(pg + 1) * P]                # [Hkv, P, d]
            assert np.array_equal(bn[b, pg, :, :d], rows.min(axis=1))
            assert np.array_equal(bn[b, pg, :, d:], rows.max(axis=1))


# ---------------------------------------------------------------- blocks per GQA group
@pytest.mark.parametrize("Hq,Hkv,G", [(8, 2, 2), (8, 1, 1), (16, 1, 1)])
def test_group_block_lists_equal_repeated_head_lists(Hq, Hkv, G):
    """A BLOCKS selection with one list per KV group gives the same output as
    the same lists repeated for every query head (bitwise), on the block-sparse
    small shapes with 4, 8 and 16 query heads per group: the group's heads
    share one staging of each chosen block, the repeated lists stage it once
    per head."""
    sp = S()
    wl = dataclasses.replace(gen.WORKLOADS["msa_prefill_small"], Hq=Hq, Hkv=Hkv, H_I=4, G_sel=G)
    say(f"[gpu] group block lists {wl.name} Hq={wl.Hq} G={wl.G_sel}")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rep = hp.idx.repeat_interleave(wl.Hq // wl.G_sel, dim=1).contiguous()
    sel = sp.selection(sp.SEL_BLOCKS, rep, window=wl.window, block_size=wl.block_size)
    o2 = torch.empty_like(hp.o)
    l2 = torch.empty_like(hp.lse)
    sp.spattn_sparse_attn_fwd(hp.q, hp.k, hp.v, hp.ctx_len, 0.0, sel, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o2, hp.o) and torch.equal(l2, hp.lse)


@pytest.mark.parametrize("R", [3, 16])
def test_group_block_pick_ties(R):
    """Per-group block selection where most blocks share one mean key (exact
    ties, ranked by block index) and a few differ by one unit in the last
    place, against the oracle's selection on the same pooled keys; many rows,
    two groups of two indexer heads."""
    import oracle as orc
    from fine_grained_top_amd.hotpath import to_device
    sp = S()
    say(f"[gpu] group block pick ties R={R}")
    B, Nq, ctx, H_I, G, d_I, bs = 2, 700, 1600, 4, 2, 64, 16
    rng = np.random.default_rng(81 + R)
    base_v = rng.standard_normal(d_I).astype(np.float32)
    K = np.tile(base_v, (B, ctx, 1))
    kst = gen.f32_to_bf16_bits(K.reshape(B, ctx, 1, d_I))
    for bb in range(B):
        for blk in rng.choice(ctx // bs, size=12, replace=False):       # a few blocks nudged by one bf16 unit
            kst[bb, blk * bs, 0, blk % d_I] = int(kst[bb, blk * bs, 0, blk % d_I]) + (1 if blk % 2 else -1)
    qst = gen.f32_to_bf16_bits(rng.standard_normal((B, Nq, H_I, d_I)).astype(np.float32))
    w = rng.random(H_I).astype(np.float32)
    q = to_device(qst, "bf16")
    k = to_device(kst, "bf16")
    wd = torch.from_numpy(w).cuda().view(1, 1, H_I).expand(B, Nq, H_I)
    ix = sp.indexer(q, k, wd, sp.SCORE_WEIGHTED_RELU, H_I // G)
    lens = [ctx, ctx - 37]
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kb = torch.empty(B, ctx // bs, 1, d_I, device="cuda")
    sp.spattn_pool_index_keys(ix, cl, bs, kb)
    out = torch.empty(B, G, Nq, R, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, G, Nq, dtype=torch.int32, device="cuda")
    sp.spattn_index_block_select(ix, kb, cl, bs, R, out, cnt)
    torch.cuda.synchronize()
    got, gc = out.cpu().numpy(), cnt.cpu().numpy()
    Kd = gen.bf16_bits_to_f32(kst).astype(np.float64)[:, :, 0]
    Qd = gen.bf16_bits_to_f32(qst).astype(np.float64)
    bad = 0
    for bb in range(B):
        nbe_all = lens[bb] // bs
        pooled = orc.pooled_blocks(Kd[bb], bs, nbe_all, "f32")
        for g in range(G):
            hs = slice(g * (H_I // G), (g + 1) * (H_I // G))
            for r in range(0, Nq, 3):
                p = lens[bb] - Nq + r
                keys = orc.keys_weighted_relu(Qd[bb, r, hs], w[hs].astype(np.float64), pooled[: (p + 1) // bs])
                want = orc.group_block_select(keys, p, bs, R)
                ok = gc[bb, g, r] == len(want) and np.array_equal(got[bb, g, r, :len(want)], want) \
                    and np.all(got[bb, g, r, len(want):] == -1)
                bad += 0 if ok else 1
    assert bad == 0, f"{bad} rows differ"


def test_quest_edge_cases():
    """Quest selection at the edges: no top pages (local pages only), more
    local pages than the context holds, contexts shorter than one page, one
    list per query head, f32."""
    import oracle as orc
    sp = S()
    say("[gpu] quest edge cases")
    B, Hq, Hkv, d, P, npg = 3, 4, 2, 64, 8, 12
    rng = np.random.default_rng(91)
    K = rng.standard_normal((B, Hkv, P * npg, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, 1, d)).astype(np.float32)
    pool = np.ascontiguousarray(K.reshape(B, Hkv, npg, P, d).transpose(0, 2, 1, 3, 4).reshape(B * npg, Hkv, P, d))
    table = np.arange(B * npg, dtype=np.int32).reshape(B, npg)
    kp, tab = torch.from_numpy(pool).cuda(), torch.from_numpy(table).cuda()
    pages = sp.kv_pages(tab, P)
    lens = [5, P * npg, 3 * P + 1]
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bnd = torch.empty(B, npg, Hkv, 2 * d, device="cuda")
    sp.spattn_quest_page_bounds(kp, pages, cl, bnd)
    qd = torch.from_numpy(q).cuda()
    for G, top, loc in ((Hkv, 0, 1), (Hkv, 3, 20), (Hq, 2, 1), (Hq, 40, 2)):
        io = torch.empty(B, G, 1, top + loc, dtype=torch.int32, device="cuda")
        cnt = torch.empty(B, G, 1, dtype=torch.int32, device="cuda")
        sp.spattn_quest_select(qd, bnd, cl, P, top, loc, io, cnt)
        torch.cuda.synchronize()
        got, gc = io.cpu().numpy(), cnt.cpu().numpy()
        hg = Hq // G
        for b in range(B):
            p = lens[b] - 1
            for g in range(G):
                Qg = q[b, g * hg:(g + 1) * hg, 0].astype(np.float64)
                want = orc.quest_select(Qg, K[b, (g * hg) // (Hq // Hkv)].astype(np.float64), p, P, top, loc)
                assert gc[b, g, 0] == len(want), (G, top, loc, b, g)
                assert np.array_equal(got[b, g, 0, :len(want)], want) and np.all(got[b, g, 0, len(want):] == -1)


def test_group_block_select_wide_rows():
    """Per-group block selection beyond the wave-per-row kernel's shape (more
    than 512 blocks, 80 blocks kept): the per-row workgroup's coarse pick."""
    import oracle as orc
    from fine_grained_top_amd.hotpath import to_device
    sp = S()
    say("[gpu] group block select, 1024 blocks, R=80")
    B, Nq, ctx, H_I, G, d_I, bs, R = 1, 40, 16384, 4, 2, 64, 16, 80
    rng = np.random.default_rng(93)
    kst = gen.f32_to_bf16_bits(rng.standard_normal((B, ctx, 1, d_I)).astype(np.float32))
    qst = gen.f32_to_bf16_bits(rng.standard_normal((B, Nq, H_I, d_I)).astype(np.float32))
    w = rng.random(H_I).astype(np.float32)
    ix = sp.indexer(to_device(qst, "bf16"), to_device(kst, "bf16"),
                    torch.from_numpy(w).cuda().view(1, 1, H_I).expand(B, Nq, H_I), sp.SCORE_WEIGHTED_RELU, H_I // G)
    kb = torch.empty(B, ctx // bs, 1, d_I, device="cuda")
    sp.spattn_pool_index_keys(ix, None, bs, kb)
    out = torch.empty(B, G, Nq, R, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, G, Nq, dtype=torch.int32, device="cuda")
    sp.spattn_index_block_select(ix, kb, None, bs, R, out, cnt)
    torch.cuda.synchronize()
    got, gc = out.cpu().numpy(), cnt.cpu().numpy()
    Kd = gen.bf16_bits_to_f32(kst).astype(np.float64)[0, :, 0]
    Qd = gen.bf16_bits_to_f32(qst).astype(np.float64)[0]
    pooled = orc.pooled_blocks(Kd, bs, ctx // bs, "f32")
    for g in range(G):
        hs = slice(g * (H_I // G), (g + 1) * (H_I // G))
        for r in range(0, Nq, 7):
            p = ctx - Nq + r
            want = orc.group_block_select(orc.keys_weighted_relu(Qd[r, hs], w[hs].astype(np.float64),
                                                                 pooled[: (p + 1) // bs]), p, bs, R)
            assert gc[0, g, r] == len(want) and np.array_equal(got[0, g, r], want), (g, r)


def test_quest_decode_full_every_row():
    """Quest selection and paged attention at the full decode shapes, every row."""
    wl = gen.WORKLOADS["quest_decode"]
    say("[gpu] generating quest_decode inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    rows = _all_rows(wl, inp)
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


def test_backward_full_size():
    """The backward at the full window + global shapes (N = 4096, 8 heads,
    tiled kernel): dq of sampled rows against the oracle's gradients, and for
    every key head the identities that hold at any size: the value gradients
    sum over keys to the sum of dO over the rows and heads that read them
    (softmax rows sum to 1), and the key gradients sum to zero (each row's dS
    sums to zero)."""
    import oracle as orc
    wl = gen.WORKLOADS["window_global_bwd"]
    say("[gpu] generating window_global_bwd inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    dq, dk, dv = hp.dq.cpu().numpy(), hp.dk.cpu().numpy(), hp.dv.cpu().numpy()
    q = orc.decode(inp["q"][0], "bf16")
    k = orc.decode(inp["k"][0], "bf16")
    v = orc.decode(inp["v"][0], "bf16")
    dO = np.asarray(inp["d_o"], dtype=np.float32).astype(np.float64)[0]
    scale = 1.0 / math.sqrt(wl.d)
    worst = 0.0
    for (_, r) in _sample_rows(wl, 24, 13):
        S_ = orc.window_global_set(r, wl.window, wl.n_global)
        for h in range(0, wl.Hq, 3):
            kvh = h // (wl.Hq // wl.Hkv)
            gq, _, _ = orc.masked_attention_grads(q[h, r][None], k[kvh, :r + 1], v[kvh, :r + 1], S_, scale,
                                                  dO[h, r][None])
            worst = max(worst, float(np.abs(dq[0, h, r] - gq[0]).max()) / max(1.0, float(np.abs(gq).max())))
    say(f"  dq relative max error {worst:.2e}")
    assert worst <= 1e-4
    g = wl.Hq // wl.Hkv
    for kvh in range(wl.Hkv):
        want_v = dO[kvh * g:(kvh + 1) * g].sum(axis=(0, 1))
        got_v = dv[0, kvh].astype(np.float64).sum(axis=0)
        assert np.abs(got_v - want_v).max() <= 1e-4 * max(1.0, float(np.abs(dv[0, kvh]).sum(axis=0).max()))
        got_k = dk[0, kvh].astype(np.float64).sum(axis=0)
        assert np.abs(got_k).max() <= 1e-4 * max(1.0, float(np.abs(dk[0, kvh]).sum(axis=0).max()))


# ---------------------------------------------------------------- every row at full size
def _golden_digests():
    import importlib.util
    import json
    import os
    here = os.path.join(os.path.dirname(__file__), "golden")
    spec = importlib.util.spec_from_file_location("make_set_digests", os.path.join(here, "make_set_digests.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(here, "set_digests.json")) as f:
        return mk, json.load(f)


def _block_digests(lists, rpb):
    import hashlib
    lists = np.ascontiguousarray(lists.astype(np.int32))
    return [hashlib.sha256(lists[i:i + rpb].tobytes()).hexdigest()[:16] for i in range(0, len(lists), rpb)]


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_sets_every_row(fused):
    """Every one of the 65,536 prefill rows: the GPU's index lists hash to the
    oracle's (digests of 256-row blocks written by tests/golden/
    make_set_digests.py); a differing block is recomputed row by row with the
    oracle to name its rows. Then O on a stratified sample of 1024+ rows that
    includes every row the top-K's redo kernel took."""
    mk, gold = _golden_digests()
    g = gold["dsa_prefill"]
    wl = gen.WORKLOADS["dsa_prefill"]
    say("[gpu] generating dsa_prefill inputs")
    inp = gen.generate(wl)
    assert mk.prefill_sha(inp) == g["input_sha256"], "the fixture was written for other inputs"
    hp = run_fused(wl, inp) if fused else run(wl, inp)
    assert hp.fused == fused
    idx = hp.idx[0, 0].cpu().numpy()
    rpb = gold["rows_per_block"]
    got = _block_digests(idx, rpb)
    bad = [i for i, (a, b) in enumerate(zip(got, g["digests"])) if a != b]
    if bad:
        mk._setup_prefill()
        for bi in bad[:2]:
            for r in range(bi * rpb, min(wl.Nq, (bi + 1) * rpb)):
                want = mk.padded(mk.prefill_row_set(r), wl.topk)
                if not np.array_equal(idx[r], want):
                    say(f"  row {r}: extra {sorted(set(idx[r]) - set(want))[:6]} missing {sorted(set(want) - set(idx[r]))[:6]}")
    say(f"  {len(got)} blocks of {rpb} rows, {len(bad)} differ")
    assert not bad
    # O parity: strata over positions, the redo rows, the needles' rows
    if fused:
        # the finalize kernel's redo flags follow the survivor lists (order
        # keys and positions, cap per row) and the counts in the workspace;
        # the cap follows from the workspace size: 4 (2 cap rows + 3 rows + chunks)
        sp = S()
        need = sp.LIB.spattn_topk_workspace(None, sp.ctypes.byref(hp.ix), wl.topk, sp.TOPK_FUSED_INDEX)
        nchunk = (wl.N + 511) // 512
        cap = (need // 4 - 3 * wl.Nq - nchunk) // (2 * wl.Nq)
        off = 4 * (2 * cap * wl.Nq + wl.Nq)
        redo = np.nonzero(hp.ws[off:off + 4 * wl.Nq].view(torch.int32).cpu().numpy())[0]
        say(f"  survivor lists of {cap} per row")
    else:
        redo = np.nonzero(hp.ws[:4 * wl.Nq].view(torch.int32).cpu().numpy())[0]
    rng = np.random.default_rng(17)
    strata = np.linspace(0, wl.Nq, 65).astype(int)
    rows = set(int(x) for x in redo)
    for a, b in zip(strata[:-1], strata[1:]):
        rows |= set(int(x) for x in rng.integers(a, b, size=16))
    rows |= {0, 1, 2047, 2048, wl.Nq - 1}
    rows |= set(int(i) for i in inp["needles"][:16, 1])
    rows = [(0, r) for r in sorted(rows)]
    say(f"  O on {len(rows)} rows ({len(redo)} redo rows: {list(redo[:8])})")
    assert len(rows) >= 1024
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)


def test_block_sparse_sets_every_row():
    """Every row of two heads of the block-sparse workload (2 x 32,768 rows):
    block lists hashed against the oracle's, by 256-row blocks."""
    mk, gold = _golden_digests()
    g = gold["block_sparse"]
    wl = gen.WORKLOADS["block_sparse"]
    say("[gpu] generating block_sparse inputs")
    inp = gen.generate(wl)
    assert mk.blocks_sha(inp) == g["input_sha256"], "the fixture was written for other inputs"
    from fine_grained_top_amd.hotpath import HotPath
    hp = HotPath(wl, inp)
    hp.block_select()
    torch.cuda.synchronize()
    rpb = gold["rows_per_block"]
    bad_all = 0
    for h in g["heads"]:
        lists = hp.idx[0, h].cpu().numpy()
        got = _block_digests(lists, rpb)
        bad = [i for i, (a, b) in enumerate(zip(got, g["digests"][str(h)])) if a != b]
        if bad:
            mk._setup_blocks()
            for bi in bad[:2]:
                for r in range(bi * rpb, min(wl.Nq, (bi + 1) * rpb)):
                    want = mk.padded(mk.blocks_row_list(h, r), wl.top_blocks)
                    if not np.array_equal(lists[r], want):
                        say(f"  head {h} row {r}: got {list(lists[r])} want {list(want)}")
        say(f"  head {h}: {len(got)} blocks of {rpb} rows, {len(bad)} differ")
        bad_all += len(bad)
    assert bad_all == 0


def test_backward_full_size_key_rows():
    """Key and value gradients element by element at the full window + global
    backward shapes, for sampled band key rows (only rows j..j+w-1 see such a
    key) and for global key 0 (every row sees it): the oracle's gradient of
    each row that sees the key, summed."""
    import oracle as orc
    wl = gen.WORKLOADS["window_global_bwd"]
    say("[gpu] generating window_global_bwd inputs")
    inp = gen.generate(wl)
    hp = run(wl, inp)
    dk, dv = hp.dk.cpu().numpy(), hp.dv.cpu().numpy()
    q = orc.decode(inp["q"][0], "bf16")
    k = orc.decode(inp["k"][0], "bf16")
    v = orc.decode(inp["v"][0], "bf16")
    dO = np.asarray(inp["d_o"], dtype=np.float32).astype(np.float64)[0]
    scale = 1.0 / math.sqrt(wl.d)
    g = wl.Hq // wl.Hkv
    worst = 0.0
    rng = np.random.default_rng(23)
    keys = [0] + [int(x) for x in rng.integers(wl.n_global, wl.N, size=3)] + [wl.N - 1]
    for kvh in (0, wl.Hkv - 1):
        for j in keys:
            rows = range(j, wl.N) if j < wl.n_global else range(j, min(wl.N, j + wl.window))
            want_k = np.zeros(wl.d)
            want_v = np.zeros(wl.d)
            for r in rows:
                S_ = orc.window_global_set(r, wl.window, wl.n_global)
                for h in range(kvh * g, (kvh + 1) * g):
                    _, gk, gv = orc.masked_attention_grads(q[h, r][None], k[kvh, :r + 1], v[kvh, :r + 1], S_,
                                                           scale, dO[h, r][None])
                    want_k += gk[j]
                    want_v += gv[j]
            ek = float(np.abs(dk[0, kvh, j] - want_k).max()) / max(1.0, float(np.abs(want_k).max()))
            ev = float(np.abs(dv[0, kvh, j] - want_v).max()) / max(1.0, float(np.abs(want_v).max()))
            worst = max(worst, ek, ev)
    say(f"  dk/dv relative max error over key rows {keys}: {worst:.2e}")
    assert worst <= 1e-4


def test_fused_rows_fall_back_when_the_sample_misleads():
    """Prefill-shaped fused selection with the pilot's sampled keys zeroed:
    every sampled score is 0, so tau does not filter; rows with more keys than
    the survivor lists hold take the redo kernel, shorter rows the lists. The
    result must still be exact on every row."""
    wl = dataclasses.replace(gen.WORKLOADS["dsa_prefill_small"], N=6000, Nq=6000, topk=256, needles=0)
    inp = gen.generate(wl)
    codes = inp["k_idx"]
    pos = np.arange(wl.N)
    codes[:, (pos % 2048) < 64, 0, :] = 0
    hp = run_fused(wl, inp)
    assert hp.fused
    rows = [(0, r) for r in list(range(0, 300, 7)) + list(range(300, wl.N, 97)) + [wl.N - 1]]
    res = oracle_rows(wl, inp, rows)
    check_sets(hp, res, rows, wl)
    check_out(hp, res, rows, 2e-3)
