"""Benchmark of the depth loop on one MI355X.

Prints one JSON line.  ``value`` is frames/s of the persistent executor on
the 5-layer bf16 depth loop at 64 rows, greedy (hidden 1024, 16 x 128 q / 8
kv heads, SwiGLU 3072, 16 positions, 15 heads of vocab 2048; seeded
synthetic N(0, 0.02) weights and N(0, 1) input hidden).  A "step" is one
frame: one cp_frame_run over all rows with inputs already resident in device
memory, timed with HIP events on the stream the frames run on.

The line also carries the 1-row latency, the sampled 64-row frame, the
10-layer variant, the per-phase executor (one launch per phase, eager and
HIP-graph replay), the weight-read roofline of the persistent kernel, the
HBM traffic measured by counters (from the committed profile summary, when it
was taken on the current kernel source) and the CPU oracle timed on the host
cores.

``--calibrate-copy`` instead runs a plain device copy of known size, for
scaling the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
H200_US_64ROWS = 2218.0         # the pages' persistent frame at 64 rows, H200 (another machine: context)
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_persistent_kernel_l5_r64.md")
COPY_BYTES = 512 * 1024 * 1024


def kernel_source_hash() -> str:
    """Hash of the device sources the counters were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "persistent_megakernel_streaming_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _time_frames(plan, io, steps, warmup, repeats, graph=False):
    """µs per frame: `repeats` runs of `steps` back-to-back frames after
    `warmup`, each bracketed by events on the stream the frames run on.
    Returns (median, min, max)."""
    import torch
    stream = torch.cuda.current_stream()
    if graph:
        g = torch.cuda.CUDAGraph()
        plan.run(io)
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
    out = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / steps)
    plan.device_status()
    return statistics.median(out), min(out), max(out)


def _cpu_baseline(cfg, w, inputs, min_seconds=10.0, max_frames=6):
    """The oracle on the host cores: whole 64-row frames until about
    `min_seconds` of CPU work (at most `max_frames`)."""
    from oracle import oracle
    ow = oracle.OracleWeights(cfg, w)
    threads = min(os.cpu_count() or 1, 16)
    n, t0 = 0, time.perf_counter()
    while n < max_frames and (n == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.run_frame(cfg, ow, inputs, n_threads=threads)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} whole {cfg.rows}-row frames ({dt:.1f} s)"}


def _stored_traffic():
    """Per-launch HBM bytes of the persistent kernel at 64 rows from the
    committed counter summary, or None if it was taken on other sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _measured_read_floor(nbytes, reps=20):
    """Best streaming-read rate of a plain device read over a working set of
    `nbytes` (a sum over a bf16 tensor that size), GB/s."""
    import torch
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        x.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        x.sum(dtype=torch.float32)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del x
    torch.cuda.empty_cache()
    return nbytes / best / 1e9


def calibrate_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="", help="comma list of p64,p1,s64,pp64,pp1,l10,floor (default all)")
    ap.add_argument("--calibrate-copy", action="store_true", help="run a plain copy of known size and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the depth loop shards by rows, one plan per GPU, and this "
              f"build runs no multi-GPU path; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    from persistent_megakernel_streaming_amd import cp, synth

    only = set(args.only.split(",")) if args.only else {"p64", "p1", "s64", "pp64", "pp1", "l10", "floor"}
    steps, warm, reps = args.steps, args.warmup, args.repeats
    cfg64 = synth.CONFIGS["l5_r64"]
    w = synth.make_weights(cfg64)
    wdev = cp.upload_weights(cfg64, w)
    res = {}
    plan = cp.Plan(cfg64, wdev, exec_mode="persistent", max_rows=64)
    info = plan.info()
    wbytes = info.weight_bytes_per_frame
    phases = info.n_phases
    if "p64" in only:
        io64 = cp.make_io(cfg64, synth.make_inputs(cfg64), logits=False)
        res["persistent_us_64"] = _time_frames(plan, io64, steps, warm, reps)
    plan.close()
    if "s64" in only:
        cs = synth.CONFIGS["l5_r64_sampled"]
        pls = cp.Plan(cs, wdev, exec_mode="persistent", max_rows=64)
        ios = cp.make_io(cs, synth.make_inputs(cs, sampled=True), logits=False)
        res["persistent_sampled_us_64"] = _time_frames(pls, ios, steps, warm, reps)
        pls.close()
    cfg1 = synth.CONFIGS["l5_r1"]
    if "p1" in only:
        plan1 = cp.Plan(cfg1, wdev, exec_mode="persistent", max_rows=1)
        io1 = cp.make_io(cfg1, synth.make_inputs(cfg1), logits=False)
        res["persistent_us_1"] = _time_frames(plan1, io1, steps, warm, reps)
        plan1.close()
    for tag, c, mr in (("pp64", cfg64, 64), ("pp1", cfg1, 1)):
        if tag in only:
            pp = cp.Plan(c, wdev, exec_mode="per_phase", max_rows=mr)
            io = cp.make_io(c, synth.make_inputs(c), logits=False)
            n = max(10, steps // 4)
            res[f"per_phase_graph_us_{mr}"] = _time_frames(pp, io, n, 3, 3, graph=True)
            res[f"per_phase_eager_us_{mr}"] = _time_frames(pp, io, n, 3, 3)
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
            res[f"l10_persistent_us_{rows}"] = _time_frames(pl, io, max(20, steps // 4), warm, 3)
            if rows == 1:
                res["l10_weight_bytes"] = pl.info().weight_bytes_per_frame
            pl.close()
        del w10
        torch.cuda.empty_cache()
    floor_gbps = _measured_read_floor(157 * 1024 * 1024) if "floor" in only else None

    us64 = res["persistent_us_64"][0] if "persistent_us_64" in res else None
    us1 = res["persistent_us_1"][0] if "persistent_us_1" in res else None
    floor_us = wbytes / (HBM_PEAK_GBPS * 1e3)
    out = {
        "metric": "depth-loop frames/sec at 64 rows (persistent kernel)",
        "value": (1e6 / us64) if us64 else None,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": us64 / 1e3 if us64 else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (H200_US_64ROWS / us64) if us64 else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "depth loop, 5 layers bf16, hidden 1024, 16x128 q / 8 kv heads, SwiGLU 3072, "
                               "16 positions, 15 heads of vocab 2048, 64 rows, greedy",
                   "rows": 64, "positions": 16, "layers": 5, "phases": phases,
                   "weight_bytes_per_frame": wbytes},
        "us_per_frame_1row": us1,
        "weight_floor_us_at_8TBps": floor_us,
        "x_floor_64rows": (us64 / floor_us) if us64 else None,
        "x_floor_1row": (us1 / floor_us) if us1 else None,
        "measured_read_GBps_157MB": floor_gbps,
        "detail_us_median_min_max": res,
        "repeats": reps,
    }
    if us64:
        achieved = wbytes / (us64 * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS, "traffic": _stored_traffic()}
    if us1:
        a1 = wbytes / (us1 * 1e-6) / 1e9
        out["roofline_1row"] = {"bound": "hbm", "achieved": a1, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": a1 / HBM_PEAK_GBPS}
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(cfg64, w, synth.make_inputs(cfg64))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
