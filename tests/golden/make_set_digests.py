"""Writes set_digests.json: digests of the oracle's index sets on every row of
the prefill token top-K workload (65,536 rows) and of two heads of the
block-sparse workload (32,768 rows each).

Run from the repository root:  python tests/golden/make_set_digests.py

Only the CPU oracle and the seeded input generator are called. Each row's
set is written as the GPU path lays it out (int32, ascending, -1 padded to
the list width); the digest of a block of consecutive rows is the first 16
hex digits of the SHA-256 of those rows' bytes in order. The inputs are
identified by the SHA-256 of the arrays the sets depend on, so a changed
generator shows up as a stale fixture rather than as a kernel mismatch.
"""
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from fine_grained_top_amd import inputs as gen  # noqa: E402
import oracle as orc  # noqa: E402

ROWS_PER_BLOCK = 256
BS_HEADS = (0, 9)            # block-sparse heads covered on every row

_G = {}


def input_sha(arrays):
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


def prefill_row_set(r):
    """The oracle's set for prefill row r (request 0, the single selection
    group), as the workload driver forms it: exact weighted-ReLU keys of the
    visible indexer keys, then the top K."""
    wl, inp, Ki = _G["wl"], _G["inp"], _G["Ki"]
    p = int(inp["ctx_len"][0]) - wl.Nq + r
    qi = orc.decode(inp["q_idx"][0, r], wl.idx_q_dtype)
    w = np.asarray(inp["w"], dtype=np.float32).astype(np.float64)
    keys = orc.keys_weighted_relu(qi, w, Ki[: p + 1])
    return orc.topk(keys, wl.topk)


def blocks_row_list(h, r):
    """The oracle's block list of head h, row r of the block-sparse workload."""
    wl, inp, Kd = _G["wl"], _G["inp"], _G["Kd"]
    p = int(inp["ctx_len"][0]) - wl.Nq + r
    qh = orc.decode(inp["q"][0, h, r], wl.dtype)
    keys = orc.keys_blocks(qh, Kd[h // (wl.Hq // wl.Hkv)], wl.block_size, orc.eligible_blocks(p, wl.block_size))
    return orc.topk(keys, wl.top_blocks)


def padded(s, width):
    out = np.full(width, -1, np.int32)
    out[: len(s)] = s
    return out


def prefill_block(bi):
    wl = _G["wl"]
    h = hashlib.sha256()
    for r in range(bi * ROWS_PER_BLOCK, min(wl.Nq, (bi + 1) * ROWS_PER_BLOCK)):
        h.update(padded(prefill_row_set(r), wl.topk).tobytes())
    return bi, h.hexdigest()[:16]


def blocks_block(args):
    head, bi = args
    wl = _G["wl"]
    h = hashlib.sha256()
    for r in range(bi * ROWS_PER_BLOCK, min(wl.Nq, (bi + 1) * ROWS_PER_BLOCK)):
        h.update(padded(blocks_row_list(head, r), wl.top_blocks).tobytes())
    return head, bi, h.hexdigest()[:16]


def _setup_prefill():
    wl = gen.WORKLOADS["dsa_prefill"]
    inp = gen.generate(wl)
    _G.update(wl=wl, inp=inp, Ki=orc.decode(inp["k_idx"][0, :, 0], wl.idx_k_dtype))
    return wl, inp


def _setup_blocks():
    wl = gen.WORKLOADS["block_sparse"]
    inp = gen.generate(wl)
    _G.update(wl=wl, inp=inp, Kd=[orc.decode(inp["k"][0, x], wl.dtype) for x in range(wl.Hkv)])
    return wl, inp


def prefill_sha(inp):
    return input_sha([inp["q_idx"], inp["k_idx"], inp["w"], inp["ctx_len"]])


def blocks_sha(inp):
    return input_sha([inp["q"], inp["k"], inp["ctx_len"]])


def main():
    workers = int(os.environ.get("WORKERS", os.cpu_count() or 4))
    out = {"about": "SHA-256 (first 16 hex digits) of the oracle's index sets, "
                    f"{ROWS_PER_BLOCK} consecutive rows per digest, each row int32 ascending, -1 padded. "
                    "Written by tests/golden/make_set_digests.py from the oracle and the seeded generator.",
           "rows_per_block": ROWS_PER_BLOCK}

    t0 = time.time()
    wl, inp = _setup_prefill()
    # the per-row path above is the workload driver's; check a few rows against it
    res = orc.run(wl, inp, [(0, r) for r in (0, 2047, 2048, 40000, wl.Nq - 1)], attention=False)
    for (b, g, r), s in res.sets.items():
        assert np.array_equal(s, prefill_row_set(r)), r
    nblk = (wl.Nq + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    dig = [None] * nblk
    with ProcessPoolExecutor(workers) as ex:
        for bi, d in ex.map(prefill_block, range(nblk), chunksize=1):
            dig[bi] = d
    out["dsa_prefill"] = {"input_sha256": prefill_sha(inp), "K": wl.topk, "digests": dig}
    print(f"dsa_prefill: {nblk} blocks in {time.time() - t0:.0f}s", flush=True)

    t0 = time.time()
    _G.clear()
    wl, inp = _setup_blocks()
    res = orc.run(wl, inp, [(0, r) for r in (63, 64, 511, 20000, wl.Nq - 1)], attention=False)
    for h in BS_HEADS:
        for r in (63, 64, 511, 20000, wl.Nq - 1):
            assert np.array_equal(res.blocks[(0, h, r)], blocks_row_list(h, r)), (h, r)
    nblk = (wl.Nq + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    dig = {h: [None] * nblk for h in BS_HEADS}
    with ProcessPoolExecutor(workers) as ex:
        for h, bi, d in ex.map(blocks_block, [(h, bi) for h in BS_HEADS for bi in range(nblk)], chunksize=1):
            dig[h][bi] = d
    out["block_sparse"] = {"input_sha256": blocks_sha(inp), "top_blocks": wl.top_blocks,
                           "heads": list(BS_HEADS), "digests": {str(h): dig[h] for h in BS_HEADS}}
    print(f"block_sparse: {len(BS_HEADS)} heads x {nblk} blocks in {time.time() - t0:.0f}s", flush=True)

    with open(os.path.join(HERE, "set_digests.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
