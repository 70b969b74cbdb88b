"""Benchmark of the depth loop on one MI355X.

Prints one JSON line.  ``value`` is frames/s of the persistent executor on
the 5-layer bf16 depth loop at 64 rows (greedy, synthetic N(0, 0.02)
weights); the line also carries the 1-row latency, the per-phase executor
(one launch per phase, eager and HIP-graph replay) for comparison, the
weight-read roofline of the persistent kernel and the CPU oracle timed on
the host cores.

A "step" is one frame: one cp_frame_run over all rows with inputs already
resident in device memory.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
H200_US_64ROWS = 2218.0         # pages' persistent-kernel frame at 64 rows (H200, real weights)


def _time_frames(plan, io, steps, warmup, graph=False):
    """Mean µs per frame over `steps` back-to-back frames (after `warmup`),
    measured with events on the stream the frames are enqueued on."""
    import torch
    stream = torch.cuda.current_stream()
    if graph:
        g = torch.cuda.CUDAGraph()
        plan.run(io)  # settle allocations before capture
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g.capture_begin()
            plan.run(io, stream=s.cuda_stream)
            g.capture_end()
        torch.cuda.synchronize()
        run = g.replay
    else:
        def run():
            plan.run(io)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    plan.device_status()
    return e0.elapsed_time(e1) * 1e3 / steps


def _cpu_baseline(cfg, w, inputs, rows_sample):
    from oracle import oracle
    ow = oracle.OracleWeights(cfg, w)
    threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.run_frame(cfg, ow, inputs, rows=list(range(rows_sample)), n_threads=threads)
    dt = time.perf_counter() - t0
    per_frame = dt * cfg.rows / rows_sample  # rows are independent: scale to all rows
    return {"value": 1.0 / per_frame, "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"one frame of {rows_sample} of the {cfg.rows} rows ({dt:.1f} s), scaled to {cfg.rows} rows",
            "s_per_frame": per_frame}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="", help="comma list: p64,p1,pp64,pp1,l10 (default all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the depth loop is sharded by rows: one plan per GPU); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from persistent_megakernel_streaming_amd import cp, synth

    only = set(args.only.split(",")) if args.only else {"p64", "p1", "pp64", "pp1", "l10"}
    cfg64 = synth.CONFIGS["l5_r64"]
    w = synth.make_weights(cfg64)
    wdev = cp.upload_weights(cfg64, w)
    res = {}
    plan = cp.Plan(cfg64, wdev, exec_mode="persistent", max_rows=64)
    info = plan.info()
    wbytes = info.weight_bytes_per_frame
    if "p64" in only:
        io64 = cp.make_io(cfg64, synth.make_inputs(cfg64), logits=False)
        res["persistent_us_64"] = _time_frames(plan, io64, args.steps, args.warmup)
    plan.close()
    cfg1 = synth.CONFIGS["l5_r1"]
    if "p1" in only:
        plan1 = cp.Plan(cfg1, wdev, exec_mode="persistent", max_rows=1)
        io1 = cp.make_io(cfg1, synth.make_inputs(cfg1), logits=False)
        res["persistent_us_1"] = _time_frames(plan1, io1, args.steps, args.warmup)
        plan1.close()
    for tag, c, mr in (("pp64", cfg64, 64), ("pp1", cfg1, 1)):
        if tag in only:
            pp = cp.Plan(c, wdev, exec_mode="per_phase", max_rows=mr)
            io = cp.make_io(c, synth.make_inputs(c), logits=False)
            res[f"per_phase_graph_us_{mr}"] = _time_frames(pp, io, max(10, args.steps // 4), 3, graph=True)
            res[f"per_phase_eager_us_{mr}"] = _time_frames(pp, io, max(10, args.steps // 4), 3)
            pp.close()
    del wdev
    torch.cuda.empty_cache()
    if "l10" in only:
        cfg10 = synth.CONFIGS["l10_r64"]
        w10 = cp.upload_weights(cfg10, synth.make_weights(cfg10))
        for rows in (1, 16, 64):
            c = cfg10.with_(rows=rows)
            pl = cp.Plan(c, w10, exec_mode="persistent", max_rows=rows)
            io = cp.make_io(c, synth.make_inputs(c), logits=False)
            res[f"l10_persistent_us_{rows}"] = _time_frames(pl, io, max(20, args.steps // 2), args.warmup)
            if rows == 1:
                res["l10_weight_bytes"] = pl.info().weight_bytes_per_frame
            pl.close()
        del w10

    us64 = res.get("persistent_us_64")
    floor_us = wbytes / (HBM_PEAK_GBPS * 1e3)
    out = {
        "metric": "depth-loop frames/sec at 64 rows (persistent kernel)",
        "value": (1e6 / us64) if us64 else None,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us64 / 1e3 if us64 else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (H200_US_64ROWS / us64) if us64 else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "depth loop, 5 layers bf16, hidden 1024, 16x128 q / 8 kv heads, SwiGLU 3072, "
                               "16 positions, 15 heads of vocab 2048, 64 rows, greedy",
                   "rows": 64, "positions": 16, "layers": 5, "phases": info.n_phases,
                   "weight_bytes_per_frame": wbytes},
        "us_per_frame_1row": res.get("persistent_us_1"),
        "floor_us_at_8TBps": floor_us,
        "x_floor_64rows": (us64 / floor_us) if us64 else None,
        "x_floor_1row": (res["persistent_us_1"] / floor_us) if "persistent_us_1" in res else None,
        "detail_us": res,
    }
    if us64:
        achieved = wbytes / (us64 * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS, "traffic": None}
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(cfg64, w, synth.make_inputs(cfg64), 16)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
