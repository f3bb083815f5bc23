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
import sqlite3

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# kernels of each stage, by name fragment; the plain, filtering and page-key
# indexer are one template whose fifth argument (0, 1, 2) tells them apart
# (followed by the chunks per workgroup and the tiles in flight per wave)
STAGES = {
    "index_topk_fused": ["fz_pilot", "1, 2, 3>(sp::IndexerParams)", "1, 1, 4>(sp::IndexerParams)", "fz_final"],
    "index_scores": ["0, 1, 4>(sp::IndexerParams)", "idx_generic", "idx_err"],
    "index_page_fused": ["2, 1, 4>(sp::IndexerParams)", "idx_err", "page_keys", "page_select"],
    "topk": ["topk_row", "topk_redo", "mt_zero", "mt_hist", "mt_collect", "mt_finalize"],
    "page_select": ["page_keys_kernel", "page_select_kernel"],
    "two_level_select": ["two_level_kernel"],
    "index_block_select": ["two_level_kernel"],
    "quest_select": ["quest_keys_kernel", "page_select_kernel"],
    "attention_bwd": ["attn_bwd_zero", "attn_bwd_generic", "attn_bwd_tile"],
    "block_select": ["pool_kernel", "block_select_kernel"],
    "attention": ["attn_index_mfma", "attn_combine", "attn_tile", "attn_generic_kernel", "bc_count", "bc_scan", "bc_table",
                  "bc_scatter", "bc_attn", "bc_combine"],
}
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
    for st, frags in STAGES.items():
        ks = [k for k in kernels if any(fr in k for fr in frags)]
        if args.stages and st not in args.stages.split(","):
            continue
        if ks:
            stages[st] = {"kernels": ks, "bytes": sum(kernels[k]["read_bytes"] + kernels[k]["write_bytes"] for k in ks)}
    out = {"workload": args.workload, "sources": sources_hash(), "fetch_scale": kf, "write_scale": kw,
           "calibration": {"bytes_each_way": CALIB_BYTES, "fetch_kib": calib_f, "write_kib": calib_w},
           "kernels": kernels, "stages": stages}
    with open(args.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(stages, indent=1))


if __name__ == "__main__":
    main()
