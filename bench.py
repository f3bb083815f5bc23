"""Benchmark: selective sparse attention hot path on one MI355X.

One step = indexer + certified top-K (one fused call; separate calls with
--unfused) -> sparse attention, for one batch of the DSA-style decode
workload (8 requests, 128K-token capacity, lengths U[98304, 131072], 32 query /
8 KV heads, d = 128, bf16 KV cache, fp8-e4m3 indexer keys, top-2048 per request
and KV group). Other workloads are selected with --workload. Inputs are
resident in HBM before timing; R replicas of every input tensor are cycled so
that consecutive steps touch different memory (the working set of one step,
~155 MB, would otherwise sit in the 256 MB last-level cache).

Prints one JSON line (rank 0) with throughput, per-stage times from HIP
events on the launch stream, the roofline of the dominant stage and the
CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn queries/sec at 128K ctx (indexer+top-K+attn); % HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_PEAK_TFS = 2500.0       # dense bf16 MFMA
F32_PEAK_TFS = 157.3         # fp32 vector


def roofline_of(a, ms):
    """Roofline entry for one stage from its algorithmic bytes/flops and time."""
    if a.get("bound") == "alu":
        ach = a["flops"] / (ms * 1e-3) / 1e12
        return {"bound": "alu", "achieved": round(ach, 2), "peak": F32_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(ach / F32_PEAK_TFS, 4), "traffic": None, "alg_flops_per_launch": a["flops"],
                "launch_ms": round(ms, 5)}
    if a.get("bound") == "mfma":
        ach = a["flops"] / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK_TFS, 4), "traffic": None, "alg_flops_per_launch": a["flops"],
                "launch_ms": round(ms, 5)}
    ach = a["bytes"] / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "alg_bytes_per_launch": a["bytes"],
            "launch_ms": round(ms, 5)}


def _paged_attention(wl, hp, lens, e, qkv_out):
    """Attention over page lists: every listed page is read whole (cut at the query position)."""
    import numpy as np
    P = wl.page_size
    pg = hp.idx.cpu().numpy().astype(np.int64)                      # [B, G, Nq, width]
    pos = np.stack([L - wl.Nq + np.arange(wl.Nq) for L in lens])[:, None, :, None]
    tok = np.clip(np.minimum(pg * P + P, pos + 1) - pg * P, 0, None) * (pg >= 0)
    sel_g = float(tok.sum())                                         # sum over (b, g, r) of |S|
    per_sel = max(1, wl.Hkv // wl.G_sel)                             # KV heads each list is gathered for
    return {"bytes": sel_g * per_sel * wl.d * e * 2 + qkv_out, "flops": 4.0 * sel_g * (wl.Hq // wl.G_sel) * wl.d,
            "bound": "hbm" if wl.Nq == 1 else "mfma"}


def algorithmic(wl, inp, hp, fused):
    """Algorithmic bytes (compulsory HBM traffic) and flops of one call of each stage."""
    import numpy as np
    from fine_grained_top_amd import metrics
    e = 2 if wl.dtype == "bf16" else 4
    lens = inp["ctx_len"].astype(np.int64)
    qkv_out = wl.B * wl.Hq * wl.Nq * wl.d * (e + 4) + wl.B * wl.Hq * wl.Nq * 4   # q in, O and LSE out
    out = {}
    if wl.kind == "msa":
        # block lists per KV group, read by the group's query heads; blocks inside the window count once
        blk = hp.idx.cpu().numpy()                                                # [B, G, Nq, nb]
        pos = np.stack([L - wl.Nq + np.arange(wl.Nq) for L in lens])[:, None, :]  # [B, 1, Nq]
        ws_ = np.maximum(0, pos - wl.window + 1)
        valid = blk >= 0
        lo = blk * wl.block_size
        in_win = np.clip(np.minimum(lo + wl.block_size, pos[..., None] + 1) - np.maximum(lo, ws_[..., None]), 0, None)
        size = (valid * wl.block_size).sum(-1) - (valid * in_win).sum(-1) + (pos - ws_ + 1)
        pairs = float(size.sum()) * (wl.Hq // wl.G_sel)
        kv = wl.B * wl.Hkv * wl.N * wl.d * e * 2
        out["attention"] = {"bytes": kv + qkv_out, "flops": 4.0 * pairs * wl.d, "bound": "mfma", "pairs": pairs}
        # block scores: float32 FMAs over (row, complete block, indexer head, dim); the compulsory
        # bytes are the block-key cache once, the indexer queries and weights, and the lists
        nbe = float(((pos[:, 0, :] + 1) // wl.block_size).sum())              # complete blocks over the rows
        out["index_block_select"] = {"bytes": wl.B * (wl.N // wl.block_size) * wl.G_k * wl.d_I * 4 + blk.size * 4
                                     + wl.B * wl.Nq * wl.H_I * (wl.d_I * 2 + 4),
                                     "flops": 2.0 * nbe * wl.H_I * wl.d_I, "rows": wl.B * wl.G_sel * wl.Nq,
                                     "bound": "alu"}
    elif wl.H_I:
        kb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.idx_k_dtype]
        pos = np.concatenate([L - wl.Nq + np.arange(wl.Nq) for L in lens])
        cand = float(np.sum(pos + 1))                      # (row, key) pairs scored per group
        keys_read = float(lens.sum()) * wl.G_k * wl.d_I * kb
        idx_bytes = wl.B * wl.G_sel * wl.Nq * wl.topk * 4
        flops_idx = 2.0 * cand * wl.H_I * wl.d_I
        score_bytes = cand * wl.G_sel * 4
        out["index_scores"] = {"bytes": keys_read + score_bytes, "flops": flops_idx,
                               "bound": "hbm" if wl.Nq == 1 else "mfma"}
        out["topk"] = {"bytes": score_bytes + idx_bytes, "rows": wl.B * wl.G_sel * wl.Nq}
        out["index_topk_fused"] = {"bytes": keys_read + idx_bytes, "flops": flops_idx,
                                   "rows": wl.B * wl.G_sel * wl.Nq, "bound": "hbm" if wl.Nq == 1 else "mfma"}
        sel = np.minimum(pos + 1, wl.topk).astype(np.float64)  # |S| per row
        gath = float(sel.sum()) * (wl.Hq // max(wl.Hq // wl.G_sel, wl.Hq // wl.Hkv)) * wl.d * e * 2
        pairs = float(sel.sum()) * wl.Hq / wl.G_sel * wl.G_sel
        flops_att = 4.0 * pairs * wl.d
        out["attention"] = {"bytes": gath + qkv_out, "flops": flops_att,
                            "bound": "hbm" if wl.Nq == 1 else "mfma"}
        if wl.kind == "dsa_two_level":
            # block keys of the complete blocks, then the candidates' token keys
            nbe = np.stack([(L - wl.Nq + np.arange(wl.Nq) + 1) // wl.block_size for L in lens])   # [B, Nq]
            nopen = np.stack([L - wl.Nq + np.arange(wl.Nq) + 1 for L in lens]) - nbe * wl.block_size
            ncand = np.minimum(nbe, wl.top_blocks) * wl.block_size + nopen
            rd = float((nbe * wl.d_I * 4 + ncand * wl.d_I * kb).sum()) * wl.G_sel
            out["two_level_select"] = {"bytes": rd + idx_bytes, "rows": wl.B * wl.G_sel * wl.Nq}
        if wl.kind == "dsa_pages":
            # page lists: every listed page is read whole (cut at the query position)
            P = wl.page_size
            width = wl.top_pages + wl.n_local
            out["page_select"] = {"bytes": score_bytes + wl.B * wl.G_sel * wl.Nq * width * 4,
                                  "rows": wl.B * wl.G_sel * wl.Nq}
            out["index_page_fused"] = {"bytes": keys_read + wl.B * wl.G_sel * wl.Nq * width * 4, "flops": flops_idx,
                                       "rows": wl.B * wl.G_sel * wl.Nq, "bound": "hbm" if wl.Nq == 1 else "mfma"}
            out["attention"] = _paged_attention(wl, hp, lens, e, qkv_out)
    elif wl.kind == "quest":
        # the bounds (min and max rows) of every candidate page of rows that rank pages, q in, page lists out
        pos = np.stack([L - wl.Nq + np.arange(wl.Nq) for L in lens])              # [B, Nq]
        npc = np.maximum(0, pos // wl.page_size + 1 - wl.n_local)
        rows = wl.B * wl.G_sel * wl.Nq
        bnd = float(np.where(npc > wl.top_pages, npc, 0).sum()) * wl.G_sel * 2 * wl.d * e
        out["quest_select"] = {"bytes": bnd + wl.B * wl.Hq * wl.Nq * wl.d * e
                               + rows * (wl.top_pages + wl.n_local) * 4, "rows": rows}
        out["attention"] = _paged_attention(wl, hp, lens, e, qkv_out)
    elif wl.kind == "window_global":
        pairs = float(metrics.window_stride_pairs(wl.N, wl.window, wl.n_global, wl.stride)) * wl.Hq * wl.B
        kv = wl.B * wl.Hkv * wl.N * wl.d * e * 2
        # a dilated stride makes every row see ~p/stride keys: the products, not the bytes, bound it
        out["attention"] = {"bytes": kv + qkv_out, "flops": 4.0 * pairs * wl.d,
                            "bound": "mfma" if wl.stride else "hbm"}
        if wl.backward:
            # q, k, v, O, dO read once; dq, dk, dv written once; five products of 2 flops per
            # (pair, dim): s = q.k, dp = dO.v and dq += ds k run on bf16 MFMA (dO and dS as exact
            # three-part splits), dk += ds q and dv += p dO in float32 FMAs; the float32 part is
            # priced against the vector peak (the roofline), the MFMA part against the bf16 peak
            gbytes = wl.B * (wl.Hq * wl.Nq * wl.d * (e + 4 + 4 + 4 + 4) + wl.Hkv * wl.N * wl.d * (2 * e + 8))
            out["attention_bwd"] = {"bytes": gbytes, "flops": 4.0 * pairs * wl.d, "bound": "alu",
                                    "mfma_flops": 6.0 * pairs * wl.d, "all_flops": 10.0 * pairs * wl.d}
    elif wl.kind == "nsa":
        # three branches: pooled entries of complete blocks, the chosen blocks' tokens, the window
        blk = hp.idx.cpu().numpy().astype(np.int64)          # [B, Hq, Nq, nb]
        p = np.arange(wl.Nq)[None, None, :, None]
        tok = np.clip(np.minimum(blk * wl.block_size + wl.block_size, p + 1) - blk * wl.block_size, 0, None)
        sel_pairs = float((tok * (blk >= 0)).sum())
        pos = np.arange(wl.Nq)
        win_pairs = float(np.minimum(pos + 1, wl.window).sum()) * wl.Hq * wl.B
        cmp_pairs = float(((pos + 1) // wl.block_size).sum()) * wl.Hq * wl.B
        kv = wl.B * wl.Hkv * wl.N * wl.d * e * 2
        out["attention"] = {"bytes": kv + qkv_out, "flops": 4.0 * (sel_pairs + win_pairs + cmp_pairs) * wl.d,
                            "bound": "mfma"}
        nbk = wl.N // wl.block_size
        elig = float(np.sum(np.minimum((np.arange(wl.Nq) + 1) // wl.block_size, nbk))) * wl.Hq * wl.B
        out["block_select"] = {"bytes": wl.B * wl.Hkv * wl.N * wl.d * e + wl.B * wl.Hq * wl.Nq * wl.d * e
                               + blk.size * 4, "flops": 2.0 * elig * wl.d, "rows": wl.B * wl.Hq * wl.Nq}
    elif wl.kind == "blocks":
        blk = hp.idx.cpu().numpy()                       # [B, Hq, Nq, nb]
        p = np.arange(wl.Nq)[None, None, :]
        ws = np.maximum(0, p - wl.window + 1)
        valid = blk >= 0
        lo = blk * wl.block_size
        in_win = np.clip(np.minimum(lo + wl.block_size, p[..., None] + 1) - np.maximum(lo, ws[..., None]), 0, None)
        size = (valid * wl.block_size).sum(-1) - (valid * in_win).sum(-1) + (p - ws + 1)
        pairs = float(size.sum())
        kv = wl.B * wl.Hkv * wl.N * wl.d * e * 2
        out["attention"] = {"bytes": kv + qkv_out, "flops": 4.0 * pairs * wl.d, "bound": "mfma",
                            "pairs": pairs}
        nbk = wl.N // wl.block_size
        elig = float(np.sum(np.minimum((np.arange(wl.Nq) + 1) // wl.block_size, nbk))) * wl.Hq * wl.B
        out["block_select"] = {"bytes": wl.B * wl.Hkv * wl.N * wl.d * e + wl.B * wl.Hq * wl.Nq * wl.d * e
                               + blk.size * 4, "flops": 2.0 * elig * wl.d, "rows": wl.B * wl.Hq * wl.Nq}
    return out


def selection_stats(wl, inp, hp):
    """Pairs the selection keeps against the causal candidates, summed over
    (request, query head, query row): coverage = sum |S| / sum |C| and the
    skipped-KV ratio 1 - coverage ("A Guide to Sparse Attention in Large
    Models", production deployment: monitor coverage and skipped KV)."""
    import numpy as np
    from fine_grained_top_amd import metrics
    lens = inp["ctx_len"].astype(np.int64)
    pos = np.stack([L - wl.Nq + np.arange(wl.Nq) for L in lens])            # [B, Nq]
    causal = float((pos + 1).sum()) * wl.Hq
    if wl.kind == "window_global":
        sel = float(metrics.window_stride_pairs(wl.N, wl.window, wl.n_global, wl.stride)) * wl.Hq * wl.B
    elif wl.kind in ("dsa_pages", "quest"):
        P = wl.page_size
        pg = hp.idx.cpu().numpy().astype(np.int64)
        tok = np.clip(np.minimum(pg * P + P, pos[:, None, :, None] + 1) - pg * P, 0, None) * (pg >= 0)
        sel = float(tok.sum()) * (wl.Hq // wl.G_sel)
    elif wl.kind in ("blocks", "nsa", "msa"):
        # chosen blocks' tokens union the window (no window: the NSA selection branch alone)
        blk = hp.idx.cpu().numpy().astype(np.int64)                            # [B, G or Hq, Nq, nb]
        p = pos[:, None, :]
        win = wl.window if wl.kind != "nsa" else 0
        ws = np.maximum(0, p - win + 1) if win else p + 1
        lo = blk * wl.block_size
        tok = np.clip(np.minimum(lo + wl.block_size, p[..., None] + 1) - lo, 0, None) * (blk >= 0)
        in_win = np.clip(np.minimum(lo + wl.block_size, p[..., None] + 1) - np.maximum(lo, ws[..., None]), 0, None)
        size = tok.sum(-1) - ((blk >= 0) * in_win).sum(-1) + (p - ws + 1)
        sel = float(size.sum()) * (wl.Hq // blk.shape[1])
    elif wl.H_I:
        cnt = hp.count.cpu().numpy().astype(np.int64) if hp.count is not None else None
        if cnt is None:
            cnt = np.broadcast_to(np.minimum(pos + 1, wl.topk)[:, None, :], (wl.B, wl.G_sel, wl.Nq))
        sel = float(cnt.sum()) * (wl.Hq // wl.G_sel)
    else:
        sel = causal
    return {"pairs_selected": sel, "pairs_causal": causal, "coverage": round(sel / causal, 6),
            "skipped_kv_ratio": round(1.0 - sel / causal, 6)}


def pct(ts):
    import numpy as np
    a = np.asarray(ts, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "median": round(float(np.median(a)), 5), "p90": round(float(np.percentile(a, 90)), 5)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_traffic(workload, stage):
    """HBM bytes per launch of a stage from the committed counter record of
    this workload, or None when there is none or the kernels changed since."""
    from fine_grained_top_amd import pmc_traffic
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources") != pmc_traffic.sources_hash() or stage not in rec.get("stages", {}):
        return None
    return rec["stages"][stage]["bytes"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsa_decode")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, copy a 1 GiB buffer 3 times (a known-size kernel for PMC scaling)")
    ap.add_argument("--unfused", action="store_true",
                    help="time separate indexer-scores and top-K calls instead of the fused call")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for {args.gpus}); the library has no sharded path, so "
              "there is nothing to run across GPUs", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fine_grained_top_amd import inputs as gen
    from fine_grained_top_amd.hotpath import HotPath

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = gen.WORKLOADS[args.workload]
    log(f"[bench] generating {wl.name} inputs")
    t0 = time.time()
    inp = gen.generate(wl)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; uploading {args.replicas} replicas")
    fused = bool(wl.H_I) and not args.unfused
    paths = [HotPath(wl, inp, fused=fused) for _ in range(args.replicas)]
    fused = paths[0].fused
    # share one workspace and one set of intermediate buffers, as one layer's call would
    base = paths[0]
    for hp in paths[1:]:
        hp.ws = base.ws
        if wl.H_I:
            hp.scores, hp.err = base.scores, base.err
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    stages = []
    if wl.kind == "msa":
        stages = [("index_block_select", lambda hp: hp.index_block_select()), ("attention", lambda hp: hp.attention())]
    elif wl.H_I and fused and wl.kind == "dsa_pages":
        stages = [("index_page_fused", lambda hp: hp.page_select_fused()), ("attention", lambda hp: hp.attention())]
    elif wl.H_I and fused:
        stages = [("index_topk_fused", lambda hp: hp.topk_fused()), ("attention", lambda hp: hp.attention())]
    elif wl.H_I and wl.kind == "dsa_two_level":
        stages = [("two_level_select", lambda hp: hp.topk_two_level()), ("attention", lambda hp: hp.attention())]
    elif wl.H_I and wl.kind == "dsa_pages":
        stages = [("index_scores", lambda hp: hp.index_scores()), ("page_select", lambda hp: hp.page_select()),
                  ("attention", lambda hp: hp.attention())]
    elif wl.H_I:
        stages = [("index_scores", lambda hp: hp.index_scores()), ("topk", lambda hp: hp.topk()),
                  ("attention", lambda hp: hp.attention())]
    elif wl.kind in ("blocks", "nsa"):
        stages = [("block_select", lambda hp: hp.block_select()), ("attention", lambda hp: hp.attention())]
    elif wl.kind == "quest":
        stages = [("quest_select", lambda hp: hp.quest_select()), ("attention", lambda hp: hp.attention())]
    else:
        stages = [("attention", lambda hp: hp.attention())]
    if wl.backward:
        stages.append(("attention_bwd", lambda hp: hp.attention_bwd()))

    def step(i, ev=None):
        hp = paths[i % len(paths)]
        for si, (_, fn) in enumerate(stages):
            if ev is not None:
                ev[si][0].record(stream)
            fn(hp)
            if ev is not None:
                ev[si][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: whole-job throughput
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps

    # per-stage HIP-event timing over a second pass of the same steps
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in stages] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms, stage_pct = {}, {}
    for si, (name, _) in enumerate(stages):
        ts = [evs[i][si][0].elapsed_time(evs[i][si][1]) for i in range(args.steps)]
        stage_ms[name] = float(np.mean(ts))
        stage_pct[name] = pct(ts)
    # one event pair around each whole step (a third pass of the same steps)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        sev[i][0].record(stream)
        step(i)
        sev[i][1].record(stream)
    torch.cuda.synchronize()
    step_pct = pct([a.elapsed_time(b) for a, b in sev])

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    queries = wl.B * wl.Nq
    lens = inp["ctx_len"].astype(np.int64)
    alg = algorithmic(wl, inp, paths[(args.steps - 1) % len(paths)], fused)
    dom = max(stage_ms, key=stage_ms.get)
    roof = None
    if dom in alg:
        roof = roofline_of(alg[dom], stage_ms[dom])
        roof["kernel"] = dom
        roof["traffic"] = measured_traffic(wl.name, dom)
    per_stage = {}
    for name, ms in stage_ms.items():
        e = {"ms": round(ms, 5), "ms_p10": stage_pct[name]["p10"], "ms_median": stage_pct[name]["median"],
             "ms_p90": stage_pct[name]["p90"]}
        if name in alg:
            a = alg[name]
            e["alg_bytes"] = a["bytes"]
            e["GB_s"] = round(a["bytes"] / (ms * 1e-3) / 1e9, 1)
            e["hbm_frac"] = round(e["GB_s"] / HBM_PEAK_GBS, 4)
            if a.get("flops"):
                e["TFLOP_s"] = round(a["flops"] / (ms * 1e-3) / 1e12, 3)
                vec = a.get("bound") == "alu" or wl.dtype != "bf16"
                e["mfma_frac" if not vec else "alu_frac"] = round(e["TFLOP_s"] / (F32_PEAK_TFS if vec else MFMA_PEAK_TFS), 4)
            if a.get("mfma_flops"):
                e["mfma_part_TFLOP_s"] = round(a["mfma_flops"] / (ms * 1e-3) / 1e12, 3)
                e["mfma_part_frac"] = round(e["mfma_part_TFLOP_s"] / MFMA_PEAK_TFS, 4)
                e["all_TFLOP_s"] = round(a["all_flops"] / (ms * 1e-3) / 1e12, 3)
            if a.get("rows"):
                e["rows_per_s"] = round(a["rows"] / (ms * 1e-3), 1)
        per_stage[name] = e

    # CPU oracle on a bounded sample (also a parity spot check of the last GPU outputs)
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle as orc
        try:
            from threadpoolctl import threadpool_info
            cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
        except Exception:
            cores = os.cpu_count()
        hp = paths[(args.steps - 1) % len(paths)]
        idx = hp.idx.cpu().numpy() if hp.idx is not None else None
        O = hp.o.cpu().numpy()
        done, t0 = 0, time.perf_counter()
        ok = True
        rows = [(b, r) for b in range(wl.B) for r in range(wl.Nq)]
        rng = np.random.default_rng(0)
        if len(rows) > 64:
            rows = [rows[i] for i in rng.choice(len(rows), 64, replace=False)]
        for (b, r) in rows:
            res = orc.run(wl, inp, [(b, r)])
            done += 1
            err = float(np.abs(O[b, :, r] - res.O[(b, r)]).max())
            ok &= err <= (1e-5 if wl.dtype == "f32" else 2e-3)
            if idx is not None and wl.kind not in ("blocks", "nsa"):
                for g in range(wl.G_sel):
                    want = res.blocks[(b, g, r)] if wl.kind in ("dsa_pages", "quest", "msa") else res.sets[(b, g, r)]
                    ok &= bool(np.array_equal(idx[b, g, r, : len(want)], want))
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": round(done / dt, 4), "unit": "queries/s", "cores": cores, "kind": "oracle",
               "sample": f"{done} of {wl.B * wl.Nq} query rows of {wl.name} (all heads and groups per row), "
                         f"{dt:.1f}s",
               "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}
        # the same oracle held to one thread, on the first rows of the sample
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                d1, t1 = 0, time.perf_counter()
                for (b, r) in rows:
                    orc.run(wl, inp, [(b, r)])
                    d1 += 1
                    if time.perf_counter() - t1 > args.cpu_seconds / 2:
                        break
                dt1 = time.perf_counter() - t1
            cpu["one_thread"] = {"value": round(d1 / dt1, 4), "unit": "queries/s", "cores": 1,
                                 "sample": f"{d1} query rows, {dt1:.1f}s"}
        except ImportError:
            cpu["one_thread"] = None
        parity = bool(ok)

    from fine_grained_top_amd import metrics
    out = {
        "metric": METRIC,
        "value": round(queries / (ms_per_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "path": (("fused indexer+page selection" if fused else "indexer scores, certified page selection")
                 + ", attention over a paged KV cache" if wl.kind == "dsa_pages" else
                 "Quest page selection from per-page key bounds (bounds formed before timing), attention over "
                 "a paged KV cache" if wl.kind == "quest" else
                 "top blocks per GQA group by the indexer on block-mean keys (block-key cache formed before "
                 "timing), block-sparse attention with the group's list" if wl.kind == "msa" else
                 "two-level block-then-token selection (block-key cache formed before timing)"
                 if wl.kind == "dsa_two_level" else
                 "fused indexer+top-K" if fused else "separate indexer and top-K calls"),
        "config": {"workload": wl.name, "B": wl.B, "ctx_capacity": wl.N, "Nq": wl.Nq, "Hq": wl.Hq,
                   "Hkv": wl.Hkv, "d": wl.d, "H_I": wl.H_I, "d_I": wl.d_I, "topk": wl.topk,
                   "idx_k_dtype": wl.idx_k_dtype, "len_range": wl.len_range, "replicas": args.replicas},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_ms": step_pct,
        "stages": per_stage,
        "selection": selection_stats(wl, inp, paths[(args.steps - 1) % len(paths)]),
        "oracle_spot_parity": parity,
        "kv_cache_gb_per_layer": round(metrics.kv_cache_memory_gb(wl.B, wl.N, wl.Hkv * wl.d, 1), 3),
    }
    if wl.page_size:
        out["config"].update({"page_size": wl.page_size, "top_pages": wl.top_pages, "n_local": wl.n_local})
    if wl.kind in ("dsa_two_level", "nsa", "msa"):
        out["config"].update({"block_size": wl.block_size, "top_blocks": wl.top_blocks})
    if wl.kind in ("msa", "nsa"):
        out["config"].update({"window": wl.window, "G_sel": wl.G_sel})
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
