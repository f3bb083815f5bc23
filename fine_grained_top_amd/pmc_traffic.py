"""HBM traffic per hot-path stage from two rocprofv3 counter runs.

Reads the FETCH_SIZE and WRITE_SIZE databases of the same bench command,
scales each counter by what it reads for the 1 GiB device copy that
`bench.py --calib-copy` runs after timing (a kernel that moves a known number
of bytes each way), sums the kernels of each stage and writes a JSON record
tagged with a hash of the kernel sources, so that bench.py reports the
traffic only while the kernels are unchanged.

    python -m fine_grained_top_amd.pmc_traffic --fetch F.db --write W.db \
        --workload dsa_decode --out profiles/dsa_decode_traffic.json
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import re
import sqlite3

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# kernels of each stage, by regular expression on the kernel name; the plain,
# filtering and page-key indexer are one template whose fifth argument (0, 1,
# 2) tells them apart
_IDX = r"idx_mfma64_kernel<\d+, \d+, \d+, (true|false), %d, "
STAGES = {
    "index_topk_fused": [r"fz_pilot", r"fz_final", r"fzr_pilot", r"fzr_final", r"fzr_redo", r"fill_u32", _IDX % 1],
    "index_scores": [_IDX % 0, r"idx_generic", r"idx_err"],
    "index_page_fused": [_IDX % 2, r"idx_err", r"page_keys", r"page_select"],
    "topk": [r"topk_row", r"topk_redo", r"mt_zero", r"mt_hist", r"mt_collect", r"mt_finalize"],
    "page_select": [r"page_keys_kernel", r"page_select_kernel"],
    "two_level_select": [r"tl_pool_kernel", r"two_level_kernel"],
    "index_block_select": [r"tl_pool_kernel", r"two_level_kernel", r"group_block_pick"],
    "quest_select": [r"quest_bounds", r"quest_keys_kernel", r"page_select_kernel"],
    "attention_bwd": [r"attn_bwd_zero", r"attn_bwd_generic", r"attn_bwd_tile", r"attn_bwd_reduce"],
    "block_select": [r"sp::pool_kernel", r"block_select_kernel"],
    "attention": [r"attn_index_mfma", r"attn_combine", r"attn_tile", r"attn_generic_kernel", r"bc_count", r"bc_scan",
                  r"bc_table", r"bc_scatter", r"bc_attn", r"bc_combine", r"nsa_pool", r"nsa_combine"],
}


def stage_kernels(stage: str, names) -> list:
    """The kernels among `names` that belong to `stage`."""
    pats = [re.compile(x) for x in STAGES.get(stage, [])]
    return [n for n in names if any(pt.search(n) for pt in pats)]


def split_setup(ks, calls):
    """(per-call kernels, setup kernels, calls of the stage): a kernel with fewer
    than half the stage's dispatches (the most common count among its kernels)
    builds per-input data once (page bounds, pooled block keys) and is not part
    of a call."""
    if not ks:
        return [], [], 0
    n = collections.Counter(calls[k] for k in ks).most_common(1)[0][0]
    return [k for k in ks if 2 * calls[k] >= n], [k for k in ks if 2 * calls[k] < n], n


CALIB_BYTES = 1 << 30


def sources_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                    glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def per_dispatch(db: str, counter: str):
    """kernel name -> list of the counter's value per dispatch (summed over instances)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, sum(counter_value) from pmc_events where counter_name=? "
                       "group by name, dispatch_id", (counter,)).fetchall()
    acc = collections.defaultdict(list)
    for name, _, v in rows:
        acc[name].append(float(v))
    return acc


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--stages", default="")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    f, w = per_dispatch(args.fetch, "FETCH_SIZE"), per_dispatch(args.write, "WRITE_SIZE")
    # the 1 GiB copies are the largest copy dispatches
    calib_f = max(v for k, vs in f.items() if "copyBuffer" in k for v in vs)
    calib_w = max(v for k, vs in w.items() if "copyBuffer" in k for v in vs)
    kf = CALIB_BYTES / (calib_f * 1024.0)
    kw = CALIB_BYTES / (calib_w * 1024.0)
    kernels = {}
    for name, vs in f.items():
        if "copyBuffer" in name:
            continue
        fk = sum(vs) / len(vs)
        wv = w.get(name, [])
        wk = sum(wv) / len(wv) if wv else 0.0
        kernels[name] = {"dispatches": len(vs), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                         "read_bytes": round(fk * 1024 * kf), "write_bytes": round(wk * 1024 * kw)}
    stages = {}
    for st in STAGES:
        ks, setup, _ = split_setup(stage_kernels(st, kernels), {k: v["dispatches"] for k, v in kernels.items()})
        if args.stages and st not in args.stages.split(","):
            continue
        if ks:
            stages[st] = {"kernels": ks, "bytes": sum(kernels[k]["read_bytes"] + kernels[k]["write_bytes"] for k in ks)}
            if setup:
                stages[st]["setup_kernels"] = setup
    out = {"workload": args.workload, "sources": sources_hash(), "fetch_scale": kf, "write_scale": kw,
           "calibration": {"bytes_each_way": CALIB_BYTES, "fetch_kib": calib_f, "write_kib": calib_w},
           "kernels": kernels, "stages": stages}
    with open(args.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(stages, indent=1))


if __name__ == "__main__":
    main()
