"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these compares the oracle with itself: each uses a library routine
(torch SDPA, numpy's correctly rounded float casts, math.fsum), a hand-worked
value, a closed form or a brute-force enumeration.
"""
import dataclasses
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from fine_grained_top_amd import inputs as gen
from fine_grained_top_amd import metrics
import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats
def test_decode_fp8_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.decode(codes, "fp8")
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[finite], ref[finite])
    assert orc.decode(np.array([0x7E], np.uint8), "fp8")[0] == 448.0
    assert orc.decode(np.array([0x01], np.uint8), "fp8")[0] == 2.0 ** -9


def test_decode_bf16_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # drop inf/nan
    mine = orc.decode(bits, "bf16")
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


def test_generator_encodings_match_torch_rounding():
    """The generator's RNE encoders agree with torch's casts (fp32 -> bf16 / fp8)."""
    x = np.random.default_rng(1).standard_normal(20000).astype(np.float32)
    x[:4] = [0.0, -0.0, 448.0, 2.0 ** -10]
    b = gen.f32_to_bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(b, tb)
    f8 = gen.f32_to_e4m3fn_bits(x)
    t8 = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f8, t8)


# ---------------------------------------------------------------- exact keys
def test_f32_nearest_matches_numpy_cast():
    """Exact RNE rounding of rationals agrees with numpy's correctly rounded
    float64 -> float32 cast on doubles (normal, subnormal and tie cases)."""
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000))
    f32 = rng.standard_normal(300).astype(np.float32)
    nxt = np.nextafter(f32, np.float32(np.inf))
    xs += list((f32.astype(np.float64) + nxt.astype(np.float64)) / 2)   # exact midpoints
    xs += [2.0 ** -149, 3 * 2.0 ** -150, 2.0 ** -150, 1.5 * 2.0 ** -149, 2.0 ** -126 * (1 - 2 ** -25)]
    for x in xs:
        assert orc.f32_nearest(Fraction(x)) == np.float32(x), x


def test_exact_keys_hand_worked_ties():
    for c in _gold("f32_rounding.json")["cases"]:
        q = np.array(c["q"])
        k = np.array(c["k"])[None, :]
        key = orc.keys_dot(q, k)[0]
        assert key == np.float32(c["f32"]), c
        assert not np.signbit(key)


def test_keys_dot_equals_fsum_rounding():
    """Random fp32 dot products: nearest float32 of the exact sum equals numpy's
    cast of math.fsum (correctly rounded double) whenever that double is not a
    float32 halfway point (never, for these draws)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal(32).astype(np.float32).astype(np.float64)
    K = rng.standard_normal((3000, 32)).astype(np.float32).astype(np.float64)
    keys = orc.keys_dot(q, K)
    ref = np.array([np.float32(math.fsum(q * K[j])) for j in range(K.shape[0])])
    assert np.array_equal(keys, ref)


def _brute_weighted_relu(Q, w, k):
    tot = Fraction(0)
    for h in range(Q.shape[0]):
        dh = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(Q[h], k))
        tot += Fraction(float(w[h])) * max(Fraction(0), dh)
    return tot


def test_keys_weighted_relu_brute_force():
    rng = np.random.default_rng(4)
    Q = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((4, 16)).astype(np.float32))).astype(np.float64)
    K = gen.e4m3fn_bits_to_f32(gen.f32_to_e4m3fn_bits(rng.standard_normal((400, 16)).astype(np.float32))).astype(np.float64)
    w = rng.random(4).astype(np.float32).astype(np.float64)
    keys = orc.keys_weighted_relu(Q, w, K)
    for j in range(K.shape[0]):
        ex = _brute_weighted_relu(Q, w, K[j])
        # compare against numpy's cast of the exact value's nearest double when unambiguous
        assert keys[j] == np.float32(float(ex))
        assert abs(float(keys[j]) - float(ex)) <= abs(float(ex)) * 2 ** -24 + 1e-300
    # a hand-worked case: heads [1,0] and [0,1], w = (0.5, 2), key (3, -1) -> 0.5*3 = 1.5
    assert orc.keys_weighted_relu(np.eye(2), np.array([0.5, 2.0]), np.array([[3.0, -1.0]]))[0] == 1.5
    # every head negative -> +0
    z = orc.keys_weighted_relu(np.eye(2), np.array([0.5, 2.0]), np.array([[-3.0, -1.0]]))[0]
    assert z == 0.0 and not np.signbit(z)


def test_keys_blocks_brute_force():
    rng = np.random.default_rng(5)
    d, bs, nb = 8, 4, 6
    q = rng.standard_normal(d)
    K = rng.standard_normal((bs * nb + 3, d))
    keys = orc.keys_blocks(q, K, bs, nb)
    for b in range(nb):
        ex = sum(Fraction(float(a)) * Fraction(float(c)) for t in range(bs)
                 for a, c in zip(q, K[b * bs + t])) / bs
        assert keys[b] == np.float32(float(ex))
        assert abs(float(keys[b]) - float(ex)) <= abs(float(ex)) * 2 ** -24 + 1e-300
    # hand-worked: q = (1, 2), block of two keys (1, 0) and (3, 1) -> ((1) + (3 + 2)) / 2 = 3
    assert orc.keys_blocks(np.array([1.0, 2.0]), np.array([[1.0, 0.0], [3.0, 1.0]]), 2, 1)[0] == 3.0


# ---------------------------------------------------------------- top-K (P-f)
def _brute_topk(keys, K):
    remaining = list(range(len(keys)))
    out = []
    for _ in range(min(K, len(keys))):
        best = remaining[0]
        for j in remaining[1:]:
            if keys[j] > keys[best]:          # strict: ties keep the lower index
                best = j
        out.append(best)
        remaining.remove(best)
    return sorted(out)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    keys = rng.integers(-3, 4, size=n).astype(np.float32)      # many ties
    keys[rng.random(n) < 0.2] = -0.0
    for K in (1, 3, n // 2 + 1, n, n + 5):
        assert list(orc.topk(keys, K)) == _brute_topk(list(keys), K)


def test_topk_equals_full_stable_sort():
    rng = np.random.default_rng(7)
    keys = rng.standard_normal(5000).astype(np.float32)
    keys[::7] = keys[3]                     # ties
    order = sorted(range(len(keys)), key=lambda j: (-float(keys[j]), j))
    assert list(orc.topk(keys, 300)) == sorted(order[:300])


# ---------------------------------------------------------------- attention
def _sdpa_causal(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()


def test_full_topk_is_causal_sdpa():
    """P-a: with K >= i+1 every row sees all past keys: equals causal SDPA (fp64)."""
    import dataclasses
    wl = dataclasses.replace(gen.WORKLOADS["tiny_topk_f32_small"], N=90, Nq=90, topk=1000, needles=0)
    inp = gen.generate(wl)
    res = orc.run(wl, inp, [(0, r) for r in range(wl.Nq)])
    q = orc.decode(inp["q"][0], "f32")
    k = orc.decode(inp["k"][0], "f32")
    v = orc.decode(inp["v"][0], "f32")
    ref = _sdpa_causal(q, k, v)[0]
    got = np.stack([res.O[(0, r)][0] for r in range(wl.Nq)])
    assert np.max(np.abs(got - ref)) < 1e-12


def _fixed_pattern_mask(n, window, stride):
    """The fixed local + dilated causal mask of 'Sparse Attention Is Reshaping
    Production AI' (Fixed Patterns): a key is kept if it is not in the future
    and either at most `window` positions back or at a multiple of `stride`."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(i + 1):
            m[i, j] = (i - j) <= window or (j % stride) == 0
    return m


def test_window_is_banded_attention():
    """P-b: window of w keys (incl. self) plus one global token == the page's
    fixed local+dilated mask with window w-1 and a stride longer than the
    sequence; attention under it equals torch SDPA with that boolean mask."""
    n, w, d = 70, 9, 16
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    # with a stride longer than the sequence only key 0 is a stride position,
    # so the page's mask is a w-key window plus one global token
    mask = _fixed_pattern_mask(n, w - 1, 10 * n)
    scale = 1 / math.sqrt(d)
    for i in range(n):
        S = orc.window_global_set(i, w, 1)
        assert np.array_equal(S, np.nonzero(mask[i])[0])
        o, _ = orc.masked_attention(q[i:i + 1], k[: i + 1], v[: i + 1], S, scale)
        # the same attention via torch with an explicit boolean mask
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[i:i + 1]), torch.from_numpy(k[: i + 1]), torch.from_numpy(v[: i + 1]),
            attn_mask=torch.from_numpy(mask[i, : i + 1][None, :])).numpy()
        assert np.max(np.abs(o - ref)) < 1e-12


def test_softmax_rows_sum_to_one():
    """P-c."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 32)) * 4
    K = rng.standard_normal((500, 32))
    V = rng.standard_normal((500, 32))
    S = np.sort(rng.choice(500, 77, replace=False))
    P = orc.softmax_rows(q, K, S, 1 / math.sqrt(32))
    assert np.max(np.abs(P.sum(axis=1) - 1)) <= 1e-12
    _, lse = orc.masked_attention(q, K, V, S, 1 / math.sqrt(32))
    z = (q @ K[S].T) / math.sqrt(32)
    assert np.max(np.abs(np.exp(z - lse[:, None]).sum(axis=1) - 1)) <= 1e-12


def test_window_global_pair_counts():
    """P-d: sum |S(i)| against the closed form, brute force and the pages' N*w + N*g."""
    g = _gold("pages_arithmetic.json")["window_global_counts"]
    for n, w, gg, expect in g["cases"]:
        assert metrics.window_global_pairs(n, w, gg) == expect
    for n, w, gg in [(12, 2, 2), (40, 7, 3), (33, 33, 0), (50, 10, 10), (16384, 512, 16), (33, 33, 2),
                     (10, 9, 5), (6, 20, 3)]:
        tot = sum(len(orc.window_global_set(p, w, gg)) for p in range(n))
        assert tot == metrics.window_global_pairs(n, w, gg)
        if n <= 50:
            brute = sum(1 for i in range(n) for j in range(i + 1) if j >= i - w + 1 or j < gg)
            assert tot == brute
        assert tot <= n * w + n * gg


def test_pages_pair_arithmetic():
    """P-e: the page's dense and window pair counts at N=128,000, w=4,096."""
    g = _gold("pages_arithmetic.json")["pairs"]
    N, w = g["N"], g["w"]
    assert round(N * N / 1e9, 1) == g["dense_pairs_billion_printed"]
    assert round(N * w / 1e9, 1) == g["window_pairs_billion_printed"]
    assert N / w == 31.25 and round(N / w) != g["ratio_printed"] and abs(N / w - g["ratio_printed"]) < 1
    assert round(g["N_small"] ** 2 / 1e6, 1) == g["entries_small_million_printed"]
    # the causal window count the oracle implies has the page's N*w as its leading term
    assert metrics.window_global_pairs(N, w, 0) == N * w - w * (w - 1) // 2


def test_kv_cache_memory_example():
    """P-l: the page's memory estimate (125 / 25 / 100 GB)."""
    g = _gold("pages_arithmetic.json")["kv_cache_gb"]
    a = g["args"]
    dense = metrics.kv_cache_memory_gb(a["batch"], a["ctx"], a["kv_dim"], a["layers"], 0.0, a["bytes"])
    sparse = metrics.kv_cache_memory_gb(a["batch"], a["ctx"], a["kv_dim"], a["layers"], 0.8, a["bytes"])
    assert dense == g["dense"] and abs(sparse - g["sparse_0.8"]) < 1e-9
    assert abs(dense - sparse - g["freed"]) < 1e-9


# ---------------------------------------------------------------- workloads
def test_tiny_needles_and_early_rows():
    """P-g and P-h on the tiny fp32 workload (full size)."""
    wl = gen.WORKLOADS["tiny_topk_f32"]
    inp = gen.generate(wl)
    rows = list(range(64)) + [int(i) for i in inp["needles"][:, 1]]
    res = orc.run(wl, inp, [(0, r) for r in rows])
    for (b, i, j) in inp["needles"]:
        assert j in res.sets[(0, 0, int(i))]
    q = orc.decode(inp["q"][0], "f32")
    k = orc.decode(inp["k"][0], "f32")
    v = orc.decode(inp["v"][0], "f32")
    ref = _sdpa_causal(q[:, :64], k[:, :64], v[:, :64])[0]
    for r in range(64):
        assert np.array_equal(res.sets[(0, 0, r)], np.arange(r + 1))
        assert np.max(np.abs(res.O[(0, r)][0] - ref[r])) < 1e-12


def test_prefill_needles_selected():
    """P-g on the DSA-style prefill workload: every planted needle is selected
    by its query row (rows of the needles only, indexer + top-K)."""
    wl = gen.WORKLOADS["dsa_prefill"]
    inp = {}
    inp["ctx_len"] = gen.lengths(wl)
    inp["q_idx"] = gen.normal(wl.seed, gen.TID["q_idx"], (wl.B, wl.Nq, wl.H_I, wl.d_I), wl.idx_q_dtype)
    inp["k_idx"] = gen.normal(wl.seed, gen.TID["k_idx"], (wl.B, wl.N, wl.G_k, wl.d_I), wl.idx_k_dtype)
    inp["w"] = gen.uniform01(wl.seed, gen.TID["w"], (wl.H_I,))
    needles = gen._plant_needles(wl, inp)
    assert len(needles) == 655
    w = inp["w"].astype(np.float64)
    for (b, i, j) in needles[:40]:
        qi = orc.decode(inp["q_idx"][b, i], "bf16")
        Ki = orc.decode(inp["k_idx"][b, : i + 1, 0], "bf16")
        S = orc.topk(orc.keys_weighted_relu(qi, w, Ki), wl.topk)
        assert j in S


def test_blocks_full_coverage_is_causal():
    """P-i: with top_blocks >= eligible blocks and window >= p+1 -> full causal."""
    import dataclasses
    wl = dataclasses.replace(gen.WORKLOADS["block_sparse_small"], N=200, Nq=200, top_blocks=10,
                             window=400, Hq=1, Hkv=1)
    inp = gen.generate(wl)
    res = orc.run(wl, inp, [(0, r) for r in range(0, 200, 7)])
    q = orc.decode(inp["q"][0], "bf16")
    k = orc.decode(inp["k"][0], "bf16")
    v = orc.decode(inp["v"][0], "bf16")
    ref = _sdpa_causal(q, k, v)[0]
    for r in range(0, 200, 7):
        assert np.array_equal(res.sets[(0, 0, r)], np.arange(r + 1))
        assert np.max(np.abs(res.O[(0, r)][0] - ref[r])) < 1e-12


def test_block_selection_brute_force():
    """Block selection on a tiny case: pooled-mean scores by exact rationals,
    ranked by brute force over all eligible blocks."""
    rng = np.random.default_rng(10)
    bs, d, n = 4, 6, 37
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    for p in (3, 4, 15, 36):
        ne = (p + 1) // bs
        ex = [sum(Fraction(float(a)) * Fraction(float(c)) for t in range(bs)
                  for a, c in zip(q, K[b * bs + t])) / bs for b in range(ne)]
        want = sorted(sorted(range(ne), key=lambda b: (-ex[b], b))[:3])
        assert list(orc.block_select(q, K, p, bs, 3)) == want


def test_gqa_equals_replicated_mha():
    """P-j: a query-head group sharing one KV head equals MHA with K/V copied."""
    rng = np.random.default_rng(11)
    d, n = 16, 50
    q = rng.standard_normal((4, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    S = np.sort(rng.choice(n, 20, replace=False))
    O, lse = orc.masked_attention(q, K, V, S, 0.25)
    for h in range(4):
        o1, l1 = orc.masked_attention(q[h:h + 1], K.copy(), V.copy(), S, 0.25)
        assert np.max(np.abs(o1[0] - O[h])) < 1e-13 and abs(l1[0] - lse[h]) < 1e-13


def test_decode_equals_last_prefill_row():
    """P-k: the decode output of a request equals the prefill output at its last row."""
    import dataclasses
    wl = gen.WORKLOADS["dsa_decode_small"]
    dec = dataclasses.replace(wl, B=1, N=700, len_range=(650, 700), topk=64)
    inp = gen.generate(dec)
    L = int(inp["ctx_len"][0])
    rd = orc.run(dec, inp, [(0, 0)])
    pre = dataclasses.replace(dec, Nq=L, len_range=None, N=L)
    pin = dict(inp)
    pin["ctx_len"] = np.array([L], np.int32)
    pin["q"] = np.zeros((1, dec.Hq, L, dec.d), inp["q"].dtype)
    pin["q"][:, :, L - 1] = inp["q"][:, :, 0]
    pin["q_idx"] = np.zeros((1, L, dec.H_I, dec.d_I), inp["q_idx"].dtype)
    pin["q_idx"][:, L - 1] = inp["q_idx"][:, 0]
    pin["k"] = inp["k"][:, :, :L]
    pin["v"] = inp["v"][:, :, :L]
    pin["k_idx"] = inp["k_idx"][:, :L]
    rp = orc.run(pre, pin, [(0, L - 1)])
    assert np.array_equal(rd.O[(0, 0)], rp.O[(0, L - 1)])
    for g in range(dec.G_sel):
        assert np.array_equal(rd.sets[(0, g, 0)], rp.sets[(0, g, L - 1)])


def test_generator_is_deterministic():
    wl = gen.WORKLOADS["dsa_decode_small"]
    a = gen.generate(wl)
    b = gen.generate(wl)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ---------------------------------------------------------------- page-granular selection
def test_page_select_hand_worked():
    g = _gold("page_select_hand.json")
    keys = np.asarray(g["keys"], dtype=np.float32)
    for c in g["select_cases"]:
        got = orc.page_select(keys, c["p"], c["P"], c["top"], c["local"])
        assert list(got) == c["pages"], c
    for c in g["set_cases"]:
        assert list(orc.pages_set(c["pages"], c["p"], c["P"])) == c["tokens"], c


@pytest.mark.parametrize("seed", range(4))
def test_page_select_one_token_pages_is_token_topk(seed):
    """With 1-token pages and no mandatory pages, page selection is token top-K."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(5, 50))
    keys = rng.integers(-3, 4, size=n).astype(np.float32)
    for p in (0, n // 3, n - 1):
        for K in (1, 4, p + 1, p + 3):
            assert list(orc.page_select(keys, p, 1, K, 0)) == _brute_topk(list(keys[:p + 1]), K)


@pytest.mark.parametrize("seed", range(6))
def test_page_select_brute_force(seed):
    """Page maxima by explicit loops, ranking by brute force, recent pages always kept."""
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 70))
    keys = rng.integers(-4, 5, size=n).astype(np.float32)       # many ties
    for P in (1, 2, 4, 8):
        for n_local in (0, 1, 2, 3):
            for top in (1, 2, 5):
                for p in sorted({0, n // 2, n - 1}):
                    last = p // P
                    cands = list(range(max(0, last + 1 - n_local)))
                    pk = []
                    for pg in cands:
                        m = None
                        for j in range(pg * P, pg * P + P):
                            if j <= p and (m is None or keys[j] > m):
                                m = keys[j]
                        pk.append(m)
                    want = _brute_topk(pk, top) + list(range(len(cands), last + 1))
                    got = orc.page_select(keys, p, P, top, n_local)
                    assert list(got) == want, (P, n_local, top, p)
                    assert len(got) == min(top, len(cands)) + (last + 1 - len(cands))


def test_pages_full_coverage_is_causal():
    """Enough pages for every row: every past token is read, which is causal SDPA."""
    import dataclasses
    wl = dataclasses.replace(gen.WORKLOADS["dsa_paged_prefill_small"], N=150, Nq=150, Hq=2, Hkv=1,
                             G_sel=1, H_I=2, top_pages=100)
    inp = gen.generate(wl)
    res = orc.run(wl, inp, [(0, r) for r in range(0, 150, 11)])
    q = orc.decode(inp["q"][0], "bf16")
    k = orc.decode(inp["k"][0], "bf16")
    v = orc.decode(inp["v"][0], "bf16")
    ref = _sdpa_causal(q, np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0))
    for r in range(0, 150, 11):
        assert np.array_equal(res.sets[(0, 0, r)], np.arange(r + 1))
        for h in range(2):
            assert np.max(np.abs(res.O[(0, r)][h] - ref[h, r])) < 1e-12


def test_paged_pool_holds_the_logical_cache():
    """The generator's page pool, read through the page table, is the logical K/V."""
    wl = gen.WORKLOADS["dsa_paged_decode_small"]
    inp = gen.generate(wl)
    P = wl.page_size
    T = inp["page_table"]
    assert sorted(T.ravel().tolist()) == list(range(T.size))
    for b in range(wl.B):
        n = int(inp["ctx_len"][b])
        for name in ("k", "v"):
            pool = inp[name + "_pages"]
            rebuilt = np.concatenate([pool[T[b, pg]] for pg in range((n + P - 1) // P)], axis=1)[:, :n]
            assert np.array_equal(rebuilt, inp[name][b, :, :n])



# ---------------------------------------------------------------- dilated stride
@pytest.mark.parametrize("stride", [1, 3, 8, 13])
def test_window_stride_is_the_pages_fixed_mask(stride):
    """Window of w keys (incl. self) plus every stride-th token == the fixed
    local + dilated mask of 'Sparse Attention Is Reshaping Production AI' with
    window w - 1; attention under it equals torch SDPA with that mask."""
    n, w, d = 60, 6, 16
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    mask = _fixed_pattern_mask(n, w - 1, stride)
    for i in range(n):
        S = orc.window_global_set(i, w, 0, stride)
        assert np.array_equal(S, np.nonzero(mask[i])[0])
        if i % 7 == 0:
            o, _ = orc.masked_attention(q[i:i + 1], k[: i + 1], v[: i + 1], S, 1 / math.sqrt(d))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[i:i + 1]), torch.from_numpy(k[: i + 1]), torch.from_numpy(v[: i + 1]),
                attn_mask=torch.from_numpy(mask[i, : i + 1][None, :])).numpy()
            assert np.max(np.abs(o - ref)) < 1e-12


def test_window_stride_pair_counts():
    """Sum of |S(i)| with window, globals and stride: oracle sets, brute force
    and the benchmark's count agree."""
    for n, w, g, s in [(40, 7, 3, 5), (64, 8, 0, 8), (50, 10, 12, 4), (33, 33, 2, 3), (45, 1, 0, 1)]:
        tot = sum(len(orc.window_global_set(p, w, g, s)) for p in range(n))
        brute = sum(1 for i in range(n) for j in range(i + 1) if j >= i - w + 1 or j < g or j % s == 0)
        assert tot == brute == metrics.window_stride_pairs(n, w, g, s)
    assert metrics.window_stride_pairs(16384, 512, 16, 0) == metrics.window_global_pairs(16384, 512, 16)


# ---------------------------------------------------------------- NSA branches
def _nsa_case(seed=14, n=40, d=8, bs=4):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))


def test_nsa_compression_of_one_token_blocks_is_causal_sdpa():
    """With one-token blocks the mean-pooled entries are the tokens, so the
    compression branch alone (gates 1, 0, 0) is causal attention."""
    q, K, V = _nsa_case()
    Q = np.random.default_rng(15).standard_normal((K.shape[0], K.shape[1]))
    ref = _sdpa_causal(Q[None], K[None], V[None])[0]
    for p in (0, 5, 39):
        o = orc.nsa_attention(Q[p], K, V, p, 1, [], 3, np.array([1.0, 0.0, 0.0]), 1 / math.sqrt(K.shape[1]))
        assert np.max(np.abs(o - ref[p])) < 1e-12


def test_nsa_pooling_is_the_block_mean():
    """Compressed entries by explicit sums over each complete block."""
    _, K, _ = _nsa_case()
    P = orc.pooled_blocks(K, 4, 9)
    for blk in range(9):
        want = [sum(K[4 * blk + t][c] for t in range(4)) / 4 for c in range(K.shape[1])]
        assert np.allclose(P[blk], want, rtol=0, atol=1e-15)
    # a block of identical rows compresses to that row (fsum is exact here)
    K2 = np.repeat(K[:1], 8, axis=0)
    assert np.array_equal(orc.pooled_blocks(K2, 8, 1)[0], K[0])


def test_block_key_cache_rounds_like_torch():
    """The float32 block-key cache (two-level and per-group selection) is the
    exact block mean rounded once to nearest-even float32, checked against
    torch's float64 -> float32 cast of math.fsum means, on rows built so some
    means sit exactly on a float32 halfway point."""
    rng = np.random.default_rng(16)
    X = rng.standard_normal((64, 5))
    # block 1: every row holds an exact float32 halfway value (a float32 plus
    # half its last unit), so the mean is that halfway value itself
    f = rng.standard_normal(5).astype(np.float32).astype(np.float64)
    half = f + np.abs(f) * 2.0 ** -24
    X[16:32] = half
    got = orc.pooled_blocks(X, 16, 4, "f32")
    means = np.array([[math.fsum(X[16 * b:16 * b + 16, c]) / 16 for c in range(5)] for b in range(4)])
    ref = torch.from_numpy(means).to(torch.float32).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(orc.pooled_blocks(X, 16, 4), means)     # no format: the exact means


def test_nsa_gates_pick_branches():
    """Each one-hot gate returns its branch alone: window attention, attention
    over the chosen blocks' tokens, compression over pooled blocks; and the
    gated sum is linear in the gates (an empty branch adds nothing)."""
    q, K, V = _nsa_case()
    sc = 1 / math.sqrt(K.shape[1])
    p, bs, w, blocks = 30, 4, 6, [1, 3, 5]
    win, _ = orc.masked_attention(q[None], K[: p + 1], V[: p + 1], np.arange(p - w + 1, p + 1), sc)
    sel_set = np.concatenate([np.arange(4 * x, 4 * x + 4) for x in blocks])
    sel, _ = orc.masked_attention(q[None], K[: p + 1], V[: p + 1], sel_set, sc)
    nc = (p + 1) // bs
    Kc = np.stack([K[4 * x: 4 * x + 4].mean(axis=0) for x in range(nc)])
    Vc = np.stack([V[4 * x: 4 * x + 4].mean(axis=0) for x in range(nc)])
    cmp_, _ = orc.masked_attention(q[None], Kc, Vc, np.arange(nc), sc)
    for g, want in (([0, 0, 1], win[0]), ([0, 1, 0], sel[0]), ([1, 0, 0], cmp_[0])):
        assert np.max(np.abs(orc.nsa_attention(q, K, V, p, bs, blocks, w, np.array(g, float), sc) - want)) < 1e-12
    g = np.array([0.2, 0.3, 0.5])
    mix = orc.nsa_attention(q, K, V, p, bs, blocks, w, g, sc)
    assert np.max(np.abs(mix - (0.2 * cmp_[0] + 0.3 * sel[0] + 0.5 * win[0]))) < 1e-12
    # before the first complete block only the window contributes
    early = orc.nsa_attention(q, K, V, 2, bs, [], w, g, sc)
    w0, _ = orc.masked_attention(q[None], K[:3], V[:3], np.arange(0, 3), sc)
    assert np.max(np.abs(early - 0.5 * w0[0])) < 1e-12



# ---------------------------------------------------------------- two-level selection
@pytest.mark.parametrize("seed", range(4))
def test_two_level_brute_force(seed):
    """Blocks ranked by brute force, candidates listed by hand, tokens ranked
    by brute force; every chosen token is a candidate."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(5, 80))
    tk = rng.integers(-4, 5, size=n).astype(np.float32)
    for bs in (1, 4, 8):
        for p in sorted({0, n // 2, n - 1}):
            nbe = (p + 1) // bs
            bk = rng.integers(-3, 4, size=nbe).astype(np.float32)
            for nb, K in ((1, 3), (2, 5), (50, 200)):
                blocks = _brute_topk(list(bk), nb)
                cand = sorted([j for b in blocks for j in range(bs * b, bs * b + bs)] + list(range(nbe * bs, p + 1)))
                order = sorted(cand, key=lambda j: (-float(tk[j]), j))[:K]
                got = orc.two_level_select(bk, tk[: p + 1], p, bs, nb, K)
                assert list(got) == sorted(order), (bs, p, nb, K)


def test_two_level_with_every_block_is_token_topk():
    """With at least as many blocks as exist the candidates are all tokens:
    two-level selection equals token top-K."""
    rng = np.random.default_rng(310)
    tk = rng.standard_normal(300).astype(np.float32)
    for p in (0, 63, 64, 200, 299):
        bk = rng.standard_normal((p + 1) // 64).astype(np.float32)
        assert np.array_equal(orc.two_level_select(bk, tk[: p + 1], p, 64, 100, 37), orc.topk(tk[: p + 1], 37))


def test_two_level_hand_worked():
    """p = 9, blocks of 4 (complete: 0 and 1, tokens 8..9 in the open block),
    block keys [5, 7]: one block keeps block 1; candidates 4..7 and 8, 9."""
    tk = np.array([9, 9, 9, 9, 1, 3, 2, 3, 0, 2], dtype=np.float32)
    got = orc.two_level_select(np.array([5, 7], np.float32), tk, 9, 4, 1, 3)
    assert list(got) == [5, 6, 7]          # keys 3, 3, then the tie of 2 at 6 and 9 goes to 6



# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("seed", range(3))
def test_attention_grads_match_torch_autograd(seed):
    """dq, dK, dV of the masked attention against torch autograd in float64
    (softmax over the visible set, everything else masked), including a
    visible set of one key and an empty one."""
    rng = np.random.default_rng(400 + seed)
    H, n, d = 3, 37, 16
    q, dO = rng.standard_normal((H, d)), rng.standard_normal((H, d))
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    scale = 1 / math.sqrt(d)
    for S in (np.sort(rng.choice(n, 11, replace=False)), np.arange(n), np.array([5]), np.array([], dtype=np.int64)):
        dq, dK, dV = orc.masked_attention_grads(q, K, V, S, scale, dO)
        if len(S) == 0:
            assert not dq.any() and not dK.any() and not dV.any()
            continue
        tq, tK, tV = (torch.tensor(x, requires_grad=True) for x in (q, K, V))
        mask = torch.zeros(n, dtype=torch.bool)
        mask[torch.from_numpy(S)] = True
        o = torch.nn.functional.scaled_dot_product_attention(tq[None], tK[None], tV[None], attn_mask=mask[None, None, :],
                                                             scale=scale)[0]
        (o * torch.from_numpy(dO)).sum().backward()
        assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
        assert np.max(np.abs(dK - tK.grad.numpy())) < 1e-12
        assert np.max(np.abs(dV - tV.grad.numpy())) < 1e-12
        # keys outside the visible set get no gradient
        outside = np.setdiff1d(np.arange(n), S)
        assert not dK[outside].any() and not dV[outside].any()


# ---------------------------------------------------------------- Quest page selection
def test_quest_hand_worked():
    """Bounds and page lists worked out by hand (tests/golden/quest_hand.json)."""
    with open(os.path.join(GOLD, "quest_hand.json")) as f:
        g = json.load(f)
    K = np.array(g["keys"], dtype=np.float64)
    heads = {k: np.array(v, dtype=np.float64) for k, v in g["heads"].items()}
    for c in g["bounds"]:
        n = K.shape[0] // c["P"]
        got = orc.quest_page_keys(heads[c["heads"]], K, c["P"], n)
        assert got.tolist() == c["keys"], c
    for c in g["select_cases"]:
        got = orc.quest_select(heads[c["heads"]], K, c["p"], c["P"], c["top"], c["local"])
        assert got.tolist() == c["pages"], c


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quest_bound_is_the_box_maximum(seed):
    """A page's bound is, summed over the group's heads, the largest value each
    head's score takes at any corner of the box the page's keys span (a linear
    function peaks at a corner of a box), found here by enumerating all 2^d
    corners in exact arithmetic; and no token of the page scores above it."""
    rng = np.random.default_rng(seed)
    d, H, P, n = 6, 2, 3, 4
    Q = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((H, d)).astype(np.float32))).astype(np.float64)
    K = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((n * P, d)).astype(np.float32))).astype(np.float64)
    keys = orc.quest_page_keys(Q, K, P, n)
    qsum = [sum(Fraction(float(Q[h, c])) for h in range(H)) for c in range(d)]
    for pg in range(n):
        rows = K[pg * P:(pg + 1) * P]
        lo, hi = rows.min(axis=0), rows.max(axis=0)
        best = None
        for mask in range(1 << d):
            x = [hi[c] if (mask >> c) & 1 else lo[c] for c in range(d)]
            vh = [sum(Fraction(float(Q[h, c])) * Fraction(float(x[c])) for c in range(d)) for h in range(H)]
            best = vh if best is None else [max(a, b) for a, b in zip(best, vh)]
        assert keys[pg] == orc.f32_nearest(sum(best))
        for t in range(P):
            s = sum(qsum[c] * Fraction(float(rows[t, c])) for c in range(d))
            assert s <= sum(best)


@pytest.mark.parametrize("seed", [3, 4])
def test_quest_one_token_pages_is_token_topk(seed):
    """With one-token pages the box is the key itself: the bound is the summed
    score (sum_h q_h) . k_j, and Quest selection is token top-K over tokens
    0..p-1 plus the query's own token."""
    rng = np.random.default_rng(seed)
    d, H, n, K_ = 16, 3, 40, 7
    Q = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((H, d)).astype(np.float32))).astype(np.float64)
    K = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))).astype(np.float64)
    qsum = Q.sum(axis=0)          # exact: three bf16 values of similar size
    for p in (5, 20, 39):
        got = orc.quest_select(Q, K, p, 1, K_, 1)
        want = np.sort(np.concatenate([orc.topk(orc.keys_dot(qsum, K[:p]), K_), [p]]))
        assert got.tolist() == want.tolist()


def test_quest_key_rounds_exact_midpoints_to_even():
    """Bounds at a float32 midpoint take the exact path and round to even."""
    Q = np.array([[1.0, 1.0]])
    for tail, want in ((2.0 ** -24, 1.0), (3 * 2.0 ** -24, 1.0 + 2.0 ** -22), (-(2.0 ** -25), 1.0), (-3 * 2.0 ** -25, 1.0 - 2.0 ** -23)):
        K = np.array([[1.0, tail], [1.0, tail]])
        got = orc.quest_page_keys(Q, K, 2, 1)
        assert got[0] == np.float32(want), (tail, got[0], want)


# ---------------------------------------------------------------- blocks per GQA group
@pytest.mark.parametrize("seed", [0, 1])
def test_group_block_select_brute_force(seed):
    """Each group's blocks: the block mean of the indexer keys rounded once to
    float32 (exact rational mean), the indexer's exact weighted-ReLU score on
    it rounded once, then a full sort by (key desc, block asc) -- all in exact
    arithmetic, against the oracle's certified path."""
    rng = np.random.default_rng(seed)
    d, H, bs, n = 8, 3, 4, 37
    to_bf = lambda x: gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)
    Q = to_bf(rng.standard_normal((H, d)))
    w = rng.random(H).astype(np.float32).astype(np.float64)
    K = to_bf(rng.standard_normal((n, d)))
    for p in (3, 4, 17, 36):
        nbe = (p + 1) // bs
        means = [[orc.f32_nearest(sum(Fraction(float(K[bi * bs + t, c])) for t in range(bs)) / bs)
                  for c in range(d)] for bi in range(nbe)]
        keys = []
        for bi in range(nbe):
            tot = Fraction(0)
            for h in range(H):
                dot = sum(Fraction(float(Q[h, c])) * Fraction(float(means[bi][c])) for c in range(d))
                tot += Fraction(float(w[h])) * max(dot, Fraction(0))
            keys.append(orc.f32_nearest(tot))
        want = sorted(sorted(range(nbe), key=lambda i: (-float(keys[i]), i))[:5])
        Kp = orc.pooled_blocks(K, bs, nbe, "f32")
        got = orc.group_block_select(orc.keys_weighted_relu(Q, w, Kp), p, bs, 5)
        assert got.tolist() == want, p


def test_group_blocks_full_coverage_is_causal_gqa():
    """Enough blocks and a window of one block: every head of every group sees
    its whole causal prefix, so the output is causal attention (torch SDPA in
    float64) with K/V shared within each group."""
    wl = dataclasses.replace(gen.WORKLOADS["msa_prefill_small"], N=130, Nq=130, top_blocks=10, window=64)
    inp = gen.generate(wl)
    rows = [(0, r) for r in range(0, 130, 7)]
    res = orc.run(wl, inp, rows)
    q = torch.from_numpy(orc.decode(inp["q"][0], "bf16"))
    k = torch.from_numpy(orc.decode(inp["k"][0], "bf16")).repeat_interleave(wl.Hq // wl.Hkv, dim=0)
    v = torch.from_numpy(orc.decode(inp["v"][0], "bf16")).repeat_interleave(wl.Hq // wl.Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    for (b, r) in rows:
        assert np.abs(res.O[(b, r)] - ref[:, r]).max() < 1e-12
        for g in range(wl.G_sel):
            assert res.sets[(b, g, r)].tolist() == list(range(r + 1))


# ---------------------------------------------------------------- per-group wiring (hand-worked)
def _wiring_case(g, G_k, score_mode, Hkv, kind="dsa_decode", **extra):
    """A decode workload of one request built from the hand-worked fixture."""
    wl = gen.Workload("wiring_hand", kind, B=1, Hq=4, Hkv=Hkv, N=5, Nq=1, d=5, dtype="f32", seed=0,
                      H_I=4, d_I=2, G_sel=2, G_k=G_k, idx_q_dtype="f32", idx_k_dtype="f32",
                      score_mode=score_mode, topk=g["K"], **extra)
    keys = [g["k_idx_group0"], g["k_idx_group1"]][:G_k]
    k_idx = np.stack([np.asarray(k, np.float32) for k in keys], axis=1)[None]        # [1, 5, G_k, 2]
    v = np.stack([(c + 1) * np.eye(5, dtype=np.float32) for c in range(Hkv)])[None]   # [1, Hkv, 5, 5]
    inp = {"ctx_len": np.array([5], np.int32), "q": np.zeros((1, 4, 1, 5), np.float32),
           "k": np.zeros((1, Hkv, 5, 5), np.float32), "v": v,
           "q_idx": np.asarray(g["q_idx"], np.float32)[None, None], "k_idx": k_idx,
           "w": np.asarray(g["w"], np.float32)}
    return wl, inp


def test_group_wiring_hand_worked():
    """Indexer heads, weights and key heads per selection group, and the query
    head -> (selection group, KV head) map, against sets and outputs worked
    out by hand (tests/golden/group_wiring_hand.json)."""
    g = _gold("group_wiring_hand.json")
    for case in g["cases"]:
        wl, inp = _wiring_case(g, case["G_k"], case["score_mode"], Hkv=4)
        res = orc.run(wl, inp, [(0, 0)], attention=False, keep_keys=True)
        for grp in range(2):
            assert res.sets[(0, grp, 0)].tolist() == case["sets"][grp], (case["name"], grp)
            assert res.keys[(0, grp, 0)].tolist() == case["scores"][grp], (case["name"], grp)
    att = g["attention"]
    for Hkv, name in ((4, "O_shared_keys_Hkv4"), (1, "O_shared_keys_Hkv1")):
        wl, inp = _wiring_case(g, 1, "weighted_relu", Hkv=Hkv)
        res = orc.run(wl, inp, [(0, 0)])
        assert np.array_equal(res.O[(0, 0)], np.asarray(att[name], np.float64)), name


def test_group_blocks_wiring_hand_worked():
    """MSA-style blocks per group with one-token blocks: each group's blocks
    are its two best tokens, plus the query's own position from the window."""
    g = _gold("group_wiring_hand.json")
    m = g["msa"]
    for G_k, tag in ((1, "shared_keys"), (2, "group_keys")):
        wl, inp = _wiring_case(g, G_k, "weighted_relu", Hkv=2, kind="msa", block_size=m["block_size"],
                               top_blocks=m["top_blocks"], window=m["window"])
        res = orc.run(wl, inp, [(0, 0)], attention=False)
        for grp in range(2):
            assert res.blocks[(0, grp, 0)].tolist() == m["blocks_" + tag][grp], (tag, grp)
            assert res.sets[(0, grp, 0)].tolist() == m["sets_" + tag][grp], (tag, grp)


def test_blocks_set_hand_worked():
    """Chosen blocks united with the window, nothing after the query."""
    for c in _gold("group_wiring_hand.json")["blocks_set"]["cases"]:
        assert orc.blocks_set(c["blocks"], c["p"], c["bs"], c["w"]).tolist() == c["set"], c
