"""Markdown summary of one bench workload: bench line, kernel trace, HBM traffic.

Inputs: the output of `bench.py --workload W` (its last line is the JSON
record), the database of a `rocprofv3 --kernel-trace --stats` run of the same
workload, and the traffic record that `pmc_traffic` wrote from the two counter
runs. The workload's description line is kept from the summary being replaced.

    python -m fine_grained_top_amd.profile_report --workload W --bench bench.log \
        --trace trace.db --traffic profiles/W_traffic.json --out profiles/W.md
"""
from __future__ import annotations

import argparse
import json
import os
import sqlite3

from fine_grained_top_amd.pmc_traffic import split_setup, stage_kernels

PROFILE_ARGS = "--steps 20 --warmup 5 --no-cpu --calib-copy"


def trace_stats(db: str):
    """kernel name -> (calls, mean duration in microseconds)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(end - start) from kernels group by name").fetchall()
    return {name: (int(n), float(avg) / 1000.0) for name, n, avg in rows}


def counter_means(db: str):
    """(kernel name, counter, mean value per dispatch) of one counter database."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, sum(counter_value) from pmc_events "
                       "group by name, dispatch_id, counter_name").fetchall()
    acc = {}
    for name, _, c, v in rows:
        acc.setdefault((name, c), []).append(float(v))
    return [(n, c, sum(v) / len(v)) for (n, c), v in acc.items()]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--bench", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--traffic", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--counters", nargs="*", default=[],
                    help="databases of further `rocprofv3 --pmc` runs of the same command (COUNTERS=DB, the"
                         " counters comma-separated)")
    args = ap.parse_args()
    w = args.workload
    line = [x for x in open(args.bench).read().splitlines() if x.startswith("{")][-1]
    bench = json.loads(line)
    traffic = json.load(open(args.traffic))
    stats = trace_stats(args.trace)
    desc = ""
    if os.path.exists(args.out):
        for x in open(args.out).read().splitlines():
            if x.startswith("Workload:"):
                desc = x
                break
    prof = f"python3 <repo>/bench.py --workload {w} {PROFILE_ARGS}"
    out = [f"# {w} — bench line, kernel trace and HBM counters", ""]
    if desc:
        out += [desc, ""]
    out += ["## Bench line", "", "Command (repository root):", "", f"    python3 bench.py --workload {w}", "", "```",
            json.dumps(bench, indent=1), "```", ""]

    # ---- kernel trace
    total = sum(n * avg for n, avg in stats.values())
    out += ["## Kernel trace", "", "Command (run from /tmp with TMPDIR=/tmp; `<repo>` is the repository root):", "",
            f"    rocprofv3 --kernel-trace --stats -d <out> -o run -- {prof}", "",
            "| kernel | calls | average µs | share |", "|---|---|---|---|"]
    for name, (n, avg) in sorted(stats.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        out.append(f"| `{name}` | {n} | {avg:.2f} | {100.0 * n * avg / total:.1f}% |")
    out += ["", "(`__amd_rocclr_copyBuffer` is the input upload and the 1 GiB calibration copy, not part of a step.)",
            ""]
    rl = bench.get("roofline") or {}
    stage = rl.get("kernel")
    if stage and stage in bench.get("stages", {}):
        ks, setup, ncall = split_setup(stage_kernels(stage, [k for k in stats if "copyBuffer" not in k]),
                                       {k: v[0] for k, v in stats.items()})
        if ks:
            per_call = sum(stats[k][0] * stats[k][1] for k in ks) / ncall
            ev = bench["stages"][stage]["ms"] * 1000.0
            out += [f"Roofline stage `{stage}` = kernels " + ", ".join(f"`{k}`" for k in ks) +
                    f": {per_call:.2f} µs of kernel time per call ({ncall} calls); the bench line's HIP-event time"
                    f" of the stage is {ev:.2f} µs.", ""]
            if setup:
                out += ["Run once per input before the timed calls (not part of the stage): " +
                        ", ".join(f"`{k}`" for k in setup) + ".", ""]

    # ---- traffic
    cal = traffic["calibration"]
    out += ["## HBM traffic (two counter runs)", "", "Commands:", "",
            f"    rocprofv3 --pmc FETCH_SIZE -d <out> -o run -- {prof}",
            f"    rocprofv3 --pmc WRITE_SIZE -d <out> -o run -- {prof}",
            f"    python3 -m fine_grained_top_amd.pmc_traffic --fetch <fetch db> --write <write db> --workload {w}"
            f" --out profiles/{w}_traffic.json",
            f"    python3 -m fine_grained_top_amd.profile_report --workload {w} --bench <bench log> --trace <trace db>"
            f" --traffic profiles/{w}_traffic.json --out profiles/{w}.md", "",
            f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {cal['fetch_kib']:.1f} KiB and WRITE_SIZE = "
            f"{cal['write_kib']:.1f} KiB per dispatch for {cal['bytes_each_way'] // 1024} KiB moved each way, so bytes"
            f" = FETCH_SIZE x {traffic['fetch_scale']:.3f} KiB and WRITE_SIZE x {traffic['write_scale']:.3f} KiB."
            f" Kernel sources hash: `{traffic['sources']}` (bench.py reports the traffic only while the sources hash"
            f" the same).", "",
            "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |",
            "|---|---|---|---|---|---|"]
    for name, k in sorted(traffic["kernels"].items()):
        out.append(f"| `{name}` | {k['dispatches']} | {k['fetch_kib']} | {k['write_kib']} | "
                   f"{k['read_bytes'] / 1e6:.2f} | {k['write_bytes'] / 1e6:.2f} |")
    out += ["", "Per stage (sum of its kernels, bytes per call):", ""]
    for st in bench.get("stages", {}):
        if st in traffic.get("stages", {}):
            out.append(f"* `{st}`: {traffic['stages'][st]['bytes'] / 1e6:.2f} MB")
    if args.counters:
        out += ["", "## Instruction and request counters", "",
                "Mean per dispatch of each kernel, one `rocprofv3 --pmc` run per line of counters:", ""]
        names, per = [], {}
        for spec in args.counters:
            ctrs, db = spec.split("=", 1)
            out.append(f"    rocprofv3 --pmc {ctrs.replace(',', ' ')} -d <out> -o run -- {prof}")
            for name, c, v in counter_means(db):
                if "copyBuffer" in name:
                    continue
                per.setdefault(name, {})[c] = v
                if c not in names:
                    names.append(c)
        out += ["", "| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        for name in sorted(per):
            out.append(f"| `{name}` | " + " | ".join(f"{per[name].get(c, float('nan')):.0f}" for c in names) + " |")
        out.append("")
    with open(args.out, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("wrote", args.out)


if __name__ == "__main__":
    main()
