#!/usr/bin/env python3
"""Benchmark: block-scored paged index top-k on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: the decode scorer (paged-K gather + MFMA GEMV + causal block
max) and the top-k selector, as one mm3_index_decode call (workloads 1, 2, 3,
5), or mm3_index_score then mm3_index_topk (chunked prefill, workloads 4 and
6; the ragged serving batch, workload 7, whose decode requests and prefill
chunks share one call).

Default workload (the JSON line's value): the high-batch long decode, the
largest single-GPU workload -- 256 requests, seq_len ~ U[32768, 131072],
query_len 4, 1 index head, topk 16, 1 init + 2 local blocks, through the
fused mm3_index_decode call.  The same run times the other workloads
(tiny decode latency, decode batch, chunked prefill, NVFP4 decode) under
"extras", each with its own roofline fraction.

Prints ONE JSON line.  Besides the contract fields it carries
  roofline      the dominant kernel (the scorer) against MI355X peak, from
                HIP-event timing of that kernel alone inside this run;
  cpu_baseline  the CPU oracle on this host, on a bounded sample, with its
                scoring and selection timed separately;
  selector      the top-k kernel's own timing;
  extras        the other workloads, measured the same way.
Inputs rotate between two copies of the page pool so that successive steps
do not hit in the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "index-K tokens scored/s + top-k rows/s; % HBM peak (decode), % MFMA (prefill)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, datasheet
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, datasheet
HEADLINE = 3                 # the largest workload that fits one GPU
EXTRAS = (1, 2, 4, 5)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE, choices=[1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--copies", type=int, default=2, help="page-pool copies rotated per step")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (step_ms_graph)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only --config (no extra workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU work for the oracle baseline")
    ap.add_argument("--burn-in-ms", type=float, default=300.0,
                    help="untimed bf16 GEMMs before each workload (clocks to their loaded state)")
    ap.add_argument("--calibrate", action="store_true",
                    help="run a 1 GiB device copy first (reference for HBM counters)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="summarise rocprofv3 CSV output in DIR and exit (no GPU)")
    ap.add_argument("--label", default="", help="label for --summarize-rocprof")
    ap.add_argument("--record-traffic", action="store_true",
                    help="with --summarize-rocprof: record counter traffic in profiles/traffic.json")
    return ap.parse_args()


PROFILES = os.path.join(ROOT, "profiles")
CALIB_BYTES = 1 << 30


# The kernels whose HBM traffic profiles/traffic.json records are the two
# scorers: their sources, the headers they include, and the build script
# (its per-source flags change their code).
SCORER_SOURCES = ("decode_score.hip", "prefill_score.hip", "mm3_device.h", "mm3_fp4.h",
                  "mm3_launch.h", "mm3_rows.h")


def kernel_source_hash() -> str:
    """Hash of the scorer kernels' sources and build flags: recorded HBM
    traffic is only reported while the scorers are the ones the counters were
    taken on."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "sparse_attention_block_paged_amd")
    for f in SCORER_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(pkg, "csrc", f), "rb").read())
    h.update(open(os.path.join(pkg, "build.py"), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    ent = rec.get(workload, {})
    if ent.get("source_hash") != kernel_source_hash() or ent.get("kernel") != kernel:
        return None
    return ent.get("bytes_per_launch")


def algorithmic(w, seq):
    """Algorithmic work of one pass.  Requests with heads * rows <= 16 go to
    the decode scorer, whose unit is bytes: every visible key once, the query
    rows, the block-table entries and the scores written.  Larger ones go to
    the prefill scorer, whose unit is flops: 2 * 128 per (row, head, visible
    key).  A request's visible keys are those up to its last row."""
    import numpy as np
    H, k = w.heads, w.topk
    key_b = w.key_bytes_per_token()
    pre = w.prefix_lens.cpu().numpy() if w.prefix_lens is not None else None
    dec = dict(k=0, q=0, t=0, s=0)
    flops = tokens = pairs = 0
    nv_all = []
    for r, (_, n) in enumerate(w.row_ranges()):
        p0 = int(pre[r]) if pre is not None else int(seq[r]) - n
        pos = p0 + np.arange(n, dtype=np.int64)
        nv = np.where(pos >= 0, pos // 128 + 1, 0)
        nv_all.append(nv)
        vis = max(0, p0 + n)
        tokens += vis
        pairs += H * int((pos + 1).clip(0).sum())
        if H * n <= 16:
            dec["k"] += vis * key_b
            dec["q"] += n * H * 256
            dec["t"] += -(-vis // 128) * 4
            dec["s"] += H * int(nv.sum()) * 4
        else:
            flops += 2 * 128 * H * int((pos + 1).clip(0).sum())
    nv = np.concatenate(nv_all) if nv_all else np.zeros(0, np.int64)
    T = w.rows
    score_bytes = H * int(nv.sum()) * 4
    out_bytes = H * T * k * 4
    scorer = dec["k"] + dec["q"] + dec["t"] + dec["s"]
    return dict(k_bytes=dec["k"], scorer_bytes=scorer, selector_bytes=score_bytes + out_bytes,
                flops=flops, tokens=tokens, rows=H * T, pairs=pairs)


def burn_in(torch, dev, ms):
    """About `ms` milliseconds of bf16 GEMMs, untimed.  After idle, the
    chip's clocks take tens of milliseconds of heavy matrix load to settle:
    the chunked-prefill scorer runs at 330-390 us per launch for the first
    ~5 ms of sustained load and at ~295 us after ~40 ms (measured, launches
    timed in groups of five from a cold start), against ~295 us from the
    first launch after these GEMMs.  Every workload is timed after the same
    sustained load, so the timings are those of a busy server."""
    if ms <= 0:
        return
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + ms / 1000.0
    c = None
    while time.perf_counter() < t_end:
        for _ in range(8):
            c = a @ b
        torch.cuda.synchronize()
    del a, b, c


def measure(cid, torch, dev, steps, warmup, ncopies, graph=False, detail=True, keep=False,
            burn_ms=0.0):
    """Time workload cid on the GPU: the whole step, then the scorer and the
    selector alone (HIP events on the stream the library launches on).
    Returns (results, workload) -- the workload only with keep, else its
    device memory is released before returning."""
    import dataclasses

    import numpy as np

    import sparse_attention_block_paged_amd as mm3
    from workloads import WORKLOADS, config

    base = config(cid, device=dev)
    seq = base.seq_lens.cpu().numpy()
    copies = [base]
    for _ in range(1, max(1, ncopies)):
        copies.append(dataclasses.replace(
            base, kdata=base.kdata.clone(),
            kscales=None if base.kscales is None else base.kscales.clone(),
            q=base.q.clone(), block_table=base.block_table.clone(),
            seq_lens=base.seq_lens.clone()))
    prefill = base.heads * base.query_len > 16
    rg = lambda w: dict(cu_seqlens_q=w.cu_seqlens_q, prefix_lens=w.prefix_lens)
    H, T = base.heads, base.rows
    outs = [torch.empty((H, T, base.topk), dtype=torch.int32, device=dev) for _ in copies]
    scores = [torch.empty((H, T, base.score_width), dtype=torch.float32, device=dev) for _ in copies]
    wss = []
    for w in copies:
        p = mm3.make_problem(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len,
                             w.sm_scale, w.kscales, **rg(w))
        n = mm3.decode_workspace_bytes(p, w.topk, False)
        wss.append(torch.empty(max(n, 256), dtype=torch.uint8, device=dev))

    def step(i):
        c = i % len(copies)
        w = copies[c]
        if prefill:
            mm3.mm3_index_score(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len,
                                w.max_seq_len, w.sm_scale, kscales=w.kscales, scores=scores[c],
                                **rg(w))
            mm3.mm3_index_topk(scores[c], w.seq_lens, w.query_len, w.max_seq_len, w.topk,
                               w.init_blocks, w.local_blocks, out=outs[c], **rg(w))
        else:
            mm3.mm3_index_decode(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len,
                                 w.max_seq_len, w.sm_scale, w.topk, w.init_blocks,
                                 w.local_blocks, kscales=w.kscales, out=outs[c],
                                 workspace=wss[c], **rg(w))

    def score_only(i):
        c = i % len(copies)
        w = copies[c]
        mm3.mm3_index_score(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len,
                            w.sm_scale, kscales=w.kscales, scores=scores[c], **rg(w))

    def topk_only(i):
        c = i % len(copies)
        w = copies[c]
        mm3.mm3_index_topk(scores[c], w.seq_lens, w.query_len, w.max_seq_len, w.topk,
                           w.init_blocks, w.local_blocks, out=outs[c], **rg(w))

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms

    def per_launch(fn, n, warm):
        """Each launch bracketed by its own events, back to back: (mean,
        [p10, p50, p90]) in ms."""
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (a, b) in enumerate(ev):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        return float(t.mean()), [round(float(x), 4) for x in np.percentile(t, [10, 50, 90])]

    burn_in(torch, dev, burn_ms)
    # whole step (the contract's timed region)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps

    # the same step captured once per pool copy and replayed: the library
    # enqueues fixed grids with no allocation, so a step captures whole
    ms_graph = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        with torch.cuda.stream(side):
            for c in range(len(copies)):
                step(c)  # eager once on the capture stream
            torch.cuda.synchronize()
            for c in range(len(copies)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(c)
                graphs.append(g)
        torch.cuda.synchronize()
        ms_graph = timed(lambda i: graphs[i % len(graphs)].replay(), steps, warmup)

    # the prefill scorer with the selection fused in (a separate entry point,
    # measured slower than the step above on these shapes): its step time
    ms_fused = None
    if prefill and not base.ragged:
        fws = []
        for w in copies:
            p = mm3.make_problem(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len,
                                 w.max_seq_len, w.sm_scale, w.kscales)
            fws.append(torch.empty(mm3.prefill_select_workspace_bytes(p, w.topk, False),
                                   dtype=torch.uint8, device=dev))

        def fused_step(i):
            c = i % len(copies)
            w = copies[c]
            mm3.mm3_index_prefill_select(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len,
                                         w.max_seq_len, w.sm_scale, w.topk, w.init_blocks,
                                         w.local_blocks, kscales=w.kscales, out=outs[c],
                                         workspace=fws[c])
        ms_fused = timed(fused_step, steps, warmup)
        del fws

    # kernels alone, on the same stream (HIP events), same inputs.  A kernel's
    # time is the loop average of back-to-back launches between one pair of
    # events; the mean of launches each bracketed by its own events, which
    # adds the events' own cost (a few microseconds), is reported beside it.
    n_k = max(steps, 20)
    ms_score = timed(score_only, n_k, 3)
    ms_topk = timed(topk_only, n_k, 3)
    _, pct_step = per_launch(step, n_k, 3)
    ms_score_each, pct_score = per_launch(score_only, n_k, 3)
    # warm: the same pool copy every launch (keys partly in the 256 MB MALL)
    ms_score_warm = timed(lambda i: score_only(0), n_k, 3) if detail else None

    alg = algorithmic(base, seq)
    if prefill and alg["scorer_bytes"]:
        # decode requests and prefill chunks in one call: both scorers run.
        # The bound is the time the two would take at peak (bytes at HBM
        # peak plus flops at MFMA peak), expressed in the dominant unit.
        t_hbm = alg["scorer_bytes"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = alg["flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        frac = (t_hbm + t_mfma) / (ms_score * 1e-3)
        roof = dict(bound="mfma", achieved=round(frac * BF16_MFMA_PEAK_TFLOPS, 2),
                    peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s", frac=round(frac, 4),
                    traffic=None,
                    kernel="decode_score_cu<%d> + prefill_score_kernel<%d, true, 0>" % (base.kfmt, base.kfmt),
                    ms=round(ms_score, 4), per_launch_flops=alg["flops"],
                    per_launch_bytes=alg["scorer_bytes"],
                    combined="(bytes/8 TB/s + flops/2.5 PFLOP/s) / measured time, over both scorers")
        step_frac = None
    elif prefill:
        achieved = alg["flops"] / (ms_score * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_MFMA_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                    traffic=recorded_traffic(base.name, "prefill_score_kernel<%d, true, 0>" % base.kfmt),
                    kernel="prefill_score_kernel<%d, true, 0>" % base.kfmt, ms=round(ms_score, 4),
                    per_launch_flops=alg["flops"])
        step_frac = None
    else:
        achieved = alg["scorer_bytes"] / (ms_score * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=recorded_traffic(base.name, "decode_score_cu<%d>" % base.kfmt),
                    kernel="decode_score_cu<%d>" % base.kfmt, ms=round(ms_score, 4),
                    per_launch_bytes=alg["scorer_bytes"])
        # the whole step (scorer + selector) against the scorer's bytes
        step_frac = round(alg["scorer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    sel_gbs = alg["selector_bytes"] / (ms_topk * 1e-3) / 1e9
    cfg = WORKLOADS[cid]
    res = dict(
        workload=base.name, config_id=cid, ms_per_step=ms, wall_s_timed=wall, ms_graph=ms_graph,
        tokens_per_s=alg["tokens"] / (ms * 1e-3), rows_per_s=alg["rows"] / (ms * 1e-3),
        roofline=roof, step_frac=step_frac, step_ms_p10_p50_p90=pct_step,
        selector=dict(kernel=mm3.mm3_index_topk_selector(scores[0], base.rows, base.max_seq_len,
                                                          base.topk),
                      ms=round(ms_topk, 4), achieved_gbs=round(sel_gbs, 1),
                      bytes=alg["selector_bytes"]),
        fused_prefill_select_ms=None if ms_fused is None else round(ms_fused, 4),
        # decode steps: one launch (small batches) or scorer + selector
        step_launches=None if prefill else mm3.mm3_index_decode_launches(
            base.q, base.kdata, base.block_table, base.seq_lens, base.query_len, base.max_seq_len,
            base.sm_scale, kscales=base.kscales, **rg(base)),
        scorer_ms_p10_p50_p90=pct_score,
        scorer_ms_each_launch_mean=round(ms_score_each, 4),
        scorer_ms_warm=None if ms_score_warm is None else round(ms_score_warm, 4),
        prefill=prefill, tokens=alg["tokens"], rows=alg["rows"],
        config={
            "workload": base.name,
            "num_reqs": base.num_reqs,
            "seq_len_range": list(cfg["lens"]),
            "sum_seq_len": alg["tokens"],
            "query_len": base.query_len if not base.ragged else "ragged, max %d" % base.query_len,
            "rows": base.rows,
            "index_heads": base.heads,
            "head_dim": 128,
            "block": 128,
            "topk": base.topk,
            "init_blocks": base.init_blocks,
            "local_blocks": base.local_blocks,
            "max_seq_len": base.max_seq_len,
            "path": "score+topk" if prefill else "fused mm3_index_decode",
            "pool_copies_rotated": len(copies),
        },
        dtype="bf16" if base.kfmt == 0 else "nvfp4-keys/bf16")
    if keep:
        return res, base
    del copies, outs, scores, wss, base
    torch.cuda.empty_cache()
    return res, None


def extra_line(res):
    """The short record of a workload timed beside the headline."""
    r = res["roofline"]
    e = {"config": res["config_id"], "ms_per_step": round(res["ms_per_step"], 5),
         "step_ms_p10_p50_p90": res["step_ms_p10_p50_p90"],
         "tokens_per_s": round(res["tokens_per_s"], 1), "rows_per_s": round(res["rows_per_s"], 1),
         "roofline": {k: r[k] for k in ("bound", "kernel", "ms", "achieved", "unit", "frac")},
         "selector": {k: res["selector"][k] for k in ("kernel", "ms")}}
    if res["step_frac"] is not None:
        e["step_frac_hbm"] = res["step_frac"]
    if res["fused_prefill_select_ms"] is not None:
        e["fused_prefill_select_ms"] = res["fused_prefill_select_ms"]
    if res["step_launches"] is not None:
        e["step_launches"] = res["step_launches"]
    if res["config_id"] == 1:
        e["us_per_step"] = round(res["ms_per_step"] * 1e3, 2)
        e["note"] = "latency only: 8 blocks of keys, too small for a roofline figure"
    return e


def main():
    args = parse()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.label, args.record_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the indexer runs on one GPU; --gpus above 1 is not supported "
              "(requests would shard across GPUs with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    # oracle worker processes for the all-cores CPU baseline, started before
    # anything touches the GPU (they import only numpy and the oracle)
    pool, cores = None, 0
    if not args.no_cpu_baseline:
        import multiprocessing as mp
        try:
            cores = len(os.sched_getaffinity(0))
        except (AttributeError, OSError):
            cores = os.cpu_count() or 1
        cores = max(1, min(16, cores))
        pool = mp.get_context("spawn").Pool(cores, initializer=_oracle_init)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate:  # known-size copy: scale reference for FETCH_SIZE / WRITE_SIZE
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    res, base = measure(args.config, torch, dev, args.steps, args.warmup, args.copies,
                        graph=args.graph, detail=True, keep=not args.no_cpu_baseline,
                        burn_ms=args.burn_in_ms)
    cpu = None
    if not args.no_cpu_baseline:
        seq = base.seq_lens.cpu().numpy()
        cpu = cpu_baseline(base, seq, args.cpu_seconds, pool, cores)
        pool.close()
        pool.join()
        del base
        torch.cuda.empty_cache()

    extras = {}
    if not args.no_extras:
        for cid in EXTRAS:
            if cid == args.config:
                continue
            r, _ = measure(cid, torch, dev, min(args.steps, 20), 3, 1 if cid == 1 else args.copies,
                           detail=False, burn_ms=args.burn_in_ms)
            extras[r["workload"]] = extra_line(r)
    copy_gbs = measured_copy_gbs(torch, dev)

    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "burn_in_ms": args.burn_in_ms,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic",
        "config": res["config"],
        "rows_per_s": round(res["rows_per_s"], 1),
        "roofline": res["roofline"],
        "step_frac_hbm": res["step_frac"],
        "selector": res["selector"],
        "step_ms_graph": None if res["ms_graph"] is None else round(res["ms_graph"], 5),
        "fused_prefill_select_ms": res["fused_prefill_select_ms"],
        "step_launches": res["step_launches"],
        "step_ms_p10_p50_p90": res["step_ms_p10_p50_p90"],
        "scorer_ms_p10_p50_p90": res["scorer_ms_p10_p50_p90"],
        "scorer_ms_each_launch_mean": res["scorer_ms_each_launch_mean"],
        "scorer_ms_warm": res["scorer_ms_warm"],
        "hbm_copy_measured_gbs": copy_gbs,
        "cpu_baseline": cpu,
        "extras": extras,
        "wall_s_timed": round(res["wall_s_timed"], 3),
    }
    print(json.dumps(line), flush=True)


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_rocprof(d, label, record):
    """Print a short summary of rocprofv3 CSV output found under d: kernel
    statistics (--kernel-trace --stats), or per-dispatch counters (--pmc),
    with FETCH_SIZE / WRITE_SIZE scaled by what the same counter reads for
    the 1 GiB calibration copy."""
    import glob
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    pmc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if stats:
        rows = _read_csv(stats[0])
        # medians from the dispatch trace: the averages include the first,
        # cold launches (page pool first touched, caches empty)
        med = {}
        trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
        if trace:
            durs = {}
            for r in _read_csv(trace[0]):
                ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                durs.setdefault(r["Kernel_Name"], []).append(ns)
            for name, v in durs.items():
                v.sort()
                med[name] = v[len(v) // 2]
        print(f"# kernel statistics ({label})")
        print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'med_us':>10s} {'min_us':>10s} {'max_us':>10s} "
              f"{'total%':>7s}")
        for r in rows[:12]:
            name = r.get("Name", r.get("KernelName", "?"))
            m = f"{med[name] / 1e3:10.2f}" if name in med else f"{'-':>10s}"
            print(f"{name[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} {m} "
                  f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} {float(r['Percentage']):7.2f}")
    if pmc:
        rows = _read_csv(pmc[0])
        per = {}
        for r in rows:
            key = (r.get("Kernel_Name", r.get("Kernel-Name", "?")), r.get("Counter_Name"))
            per.setdefault(key, []).append(float(r["Counter_Value"]))
        counters = sorted({k[1] for k in per})
        print(f"# per-dispatch counters ({label}); mean over dispatches")
        # the three calibration copies are the largest copy dispatches when the
        # run uses --copies 1 (no pool clone); take their median
        calib = {}
        for (kern, cname), vals in sorted(per.items()):
            if "copyBuffer" in kern and cname in ("FETCH_SIZE", "WRITE_SIZE"):
                top = sorted(vals)[-3:]
                calib[cname] = top[len(top) // 2]
        for (kern, cname), vals in sorted(per.items()):
            mean = sum(vals) / len(vals)
            extra = ""
            if cname in calib and calib[cname] > 0:
                scale = (CALIB_BYTES / 1024.0) / calib[cname]
                extra = f"  scaled bytes {mean * 1024 * scale:.4g} (copy scale {scale:.4f})"
            print(f"{kern[:60]:60s} {cname:14s} n={len(vals):4d} mean={mean:14.1f}{extra}")
        if record:
            path = os.path.join(PROFILES, "traffic.json")
            rec = json.load(open(path)) if os.path.exists(path) else {}
            for (kern, cname), vals in per.items():
                short = kern.split("(")[0].replace("void ", "").replace("mm3::", "")
                # the scorers bench.py times: the split-K decode scorer and the
                # prefill scorer without the fused selection
                if not (short.startswith("decode_score_cu")
                        or (short.startswith("prefill_score_kernel") and short.endswith(", 0>"))):
                    continue
                if cname not in calib:
                    continue
                scale = (CALIB_BYTES / 1024.0) / calib[cname]
                ent = rec.setdefault(label, {})
                ent["kernel"] = short
                ent["source_hash"] = kernel_source_hash()
                ent.setdefault("counters", {})[cname] = sum(vals) / len(vals) * 1024 * scale
                ent["bytes_per_launch"] = round(sum(ent["counters"].values()))
            json.dump(rec, open(path, "w"), indent=1, sort_keys=True)
            print(f"recorded -> {path}")


def measured_copy_gbs(torch, dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy of 1 GiB: bytes read + written per second (GB/s),
    the practical counterpart of the 8 TB/s datasheet figure."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def _oracle_run(a, rows_loc, topk, I, L, width):
    """The oracle's two stages on one task: (scoring seconds, selection
    seconds)."""
    import oracle
    t0 = time.perf_counter()
    s = oracle.block_scores(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"], a["block_table"],
                            a["seq_lens"], a["query_len"], a["sm_scale"], width, rows=rows_loc,
                            cu_seqlens_q=a["cu_seqlens_q"], prefix_lens=a["prefix_lens"])
    t1 = time.perf_counter()
    oracle.topk(s, a["seq_lens"], a["query_len"], topk, I, L, rows=rows_loc,
                cu_seqlens_q=a["cu_seqlens_q"], prefix_lens=a["prefix_lens"])
    return t1 - t0, time.perf_counter() - t1


def _oracle_job(job):
    """One task in a worker process (no torch, no GPU): (worker pid, scoring
    seconds, selection seconds)."""
    return (os.getpid(), *_oracle_run(*job))


def _oracle_init():
    import oracle
    oracle.build(force=False)


def _rates(tok, rows, t_score, t_sel, cores, kind_sample):
    return {"value": round(tok / (t_score + t_sel), 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "sample": kind_sample,
            "scoring": {"value": round(tok / t_score, 1), "unit": "tokens/s",
                        "seconds": round(t_score, 3)},
            "selection": {"value": round(rows / t_sel, 1), "unit": "rows/s",
                          "seconds": round(t_sel, 3)}}


def cpu_baseline_all_cores(tasks, pool, cores):
    """The same oracle tasks on the host cores this process may use (16 at
    most), one task at a time per worker process; the workers never touch the
    GPU.  The whole-path time is the busiest worker's time inside the oracle:
    shipping a request's pages to a worker process is not the oracle's work
    (the transfer-inclusive wall time is reported beside it).  Each stage's
    time is its seconds summed over the workers, divided by the workers
    used."""
    tok = sum(t[1] for t in tasks)
    rows = sum(t[2] for t in tasks)
    t0 = time.perf_counter()
    res = pool.map(_oracle_job, [t[0] for t in tasks], chunksize=1)
    wall = time.perf_counter() - t0
    busy = {}
    for pid, ts, tl in res:
        b = busy.setdefault(pid, [0.0, 0.0])
        b[0] += ts
        b[1] += tl
    n = len(busy)
    el = max(sum(v) for v in busy.values())
    ts = sum(v[0] for v in busy.values()) / n
    tl = sum(v[1] for v in busy.values()) / n
    out = _rates(tok, rows, ts, tl, cores,
                 f"the same {len(tasks)} tasks over {n} of {cores} processes; busiest worker "
                 f"{el:.2f} s in the oracle, {wall:.2f} s wall with the transfers; stage times "
                 f"averaged over the workers")
    out["value"] = round(tok / el, 1)
    return out


def _hash_arrays(h, a):
    for k in ("q_bits", "kdata", "kscales", "block_table", "seq_lens", "cu_seqlens_q",
              "prefix_lens"):
        v = a.get(k)
        if v is not None:
            h.update(k.encode())
            h.update(memoryview(v).cast("B") if v.flags.c_contiguous else v.tobytes())


def cpu_baseline(w, seq, seconds, pool=None, cores=0):
    """The oracle as it is (single-threaded C, fp64) on this host, on the same
    workload, about `seconds` of work: block scores, then the selection, each
    timed on its own.  Requests of up to 64 rows are done whole, in order;
    longer ones (prefill chunks) in passes of 16 rows spread over the
    request, one pass over every request at a time, until the time is used.
    Work is counted in the metric's units: a request's visible keys times the
    fraction of its rows done (scoring), and (head, row) pairs selected
    (selection).  The sampled inputs are hashed (sha256)."""
    import hashlib

    from workloads import host_subset
    ranges = w.row_ranges()
    arrays = {}
    h = hashlib.sha256()
    tasks, tok, rows_sel, t_score, t_sel, passes = [], 0.0, 0, 0.0, 0.0, 0
    while t_score + t_sel < seconds:
        progressed = False
        for r in range(w.num_reqs):
            n = ranges[r][1]
            if n == 0:
                continue
            stride = max(1, n // 16) if n > 64 else 1
            if passes >= stride:
                continue  # every row of this request is done
            if r not in arrays:
                arrays[r] = host_subset(w, [r])[0]
                _hash_arrays(h, arrays[r])
            a = arrays[r]
            rows_loc = list(range(passes, n, stride)) if n > 64 else None
            ts, tl = _oracle_run(a, rows_loc, w.topk, w.init_blocks, w.local_blocks, w.score_width)
            t_score += ts
            t_sel += tl
            nrows = n if rows_loc is None else len(rows_loc)
            vis = (int(a["prefix_lens"][0]) + n) if a["prefix_lens"] is not None else int(seq[r])
            t_tok = vis * nrows / n
            tok += t_tok
            rows_sel += nrows * w.heads
            tasks.append(((a, rows_loc, w.topk, w.init_blocks, w.local_blocks, w.score_width),
                          t_tok, nrows * w.heads))
            progressed = True
            if t_score + t_sel >= seconds:
                break
        passes += 1
        if not progressed:
            break
    reqs = len({id(t[0][0]) for t in tasks})
    res = _rates(tok, rows_sel, t_score, t_sel, 1,
                 f"{len(tasks)} tasks over {reqs} of {w.num_reqs} requests (whole requests up to "
                 f"64 rows; longer ones in passes of 16 rows), {int(tok)} tokens-equivalent, "
                 f"{rows_sel} (head, row) pairs, {t_score + t_sel:.1f} s, single-threaded fp64 C "
                 f"oracle")
    res["inputs_sha256"] = h.hexdigest()
    res["host_cpus"] = os.cpu_count()
    res["host_cpu_model"] = host_cpu_model()
    if pool is not None:
        try:
            res["all_cores"] = cpu_baseline_all_cores(tasks, pool, cores)
        except Exception as e:  # the single-threaded figure stands on its own
            res["all_cores"] = {"error": f"{type(e).__name__}: {e}"}
    return res


def host_cpu_model() -> str:
    """The host processor's model name, from /proc/cpuinfo ("" where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


if __name__ == "__main__":
    main()
