"""Benchmark of the depth loop on one MI355X.

Prints one JSON line.  ``value`` is frames/s of the persistent executor on
the 5-layer bf16 depth loop at 64 rows, greedy (hidden 1024, 16 x 128 q / 8
kv heads, SwiGLU 3072, 16 positions, 15 heads of vocab 2048; seeded
synthetic N(0, 0.02) weights and N(0, 1) input hidden).  A "step" is one
frame: one cp_frame_run over all rows with inputs already resident in device
memory, timed with HIP events on the stream the frames run on.

The line also carries the 1-row latency, per-frame p50 / p99, cold frames
(the Infinity Cache scrubbed by a 512 MiB read before each), the sampled
64-row frame, the 10-layer variant, the per-phase executor (one launch per
phase, eager and HIP-graph replay), the weight-read roofline of the
persistent kernel against the 8 TB/s spec and against a measured floor (a
plain HIP read kernel over a working set of the layer weights' size), the
empty-chain hand-off floor, the traffic measured by counters (from the
committed profile summary, when it was taken on the current kernel source)
and the CPU oracle timed on the host cores.  The pages' H200 figures are
listed as context only; there is no baseline for this metric on MI355X.

``--trace DIR`` instead writes traced 64- and 1-row frames (decoded split and
raw stamps); ``--calibrate-copy`` runs a plain device copy of known size, for
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


def _per_frame_us(plan, io, n, scrub=None):
    """µs of each of n frames, each bracketed by its own events (p50/p99).
    With `scrub` (a device buffer), a plain read of it runs before every
    frame, outside the events, to evict the weights from the Infinity Cache
    (cold frames)."""
    import torch
    from persistent_megakernel_streaming_amd import cp
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for _ in range(3):
        plan.run(io)
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if scrub is not None:
            cp.stream_read(scrub, sink)
        e0.record(stream)
        plan.run(io)
        e1.record(stream)
    torch.cuda.synchronize()
    plan.device_status()
    return np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_threads():
    """Host threads the oracle may use: OMP_NUM_THREADS where set (the host's
    share of cores), else every core."""
    n = os.environ.get("OMP_NUM_THREADS")
    return max(1, int(n)) if n and n.isdigit() else (os.cpu_count() or 1)


def _cpu_baseline(cfg, w, inputs, min_seconds=10.0, max_frames=4):
    """The oracle as it stands on the host cores: whole frames of the timed
    workload with every host thread until about `min_seconds` of work (at
    most `max_frames`), and one-row frames on one thread for the
    single-thread figure."""
    from oracle import oracle
    ow = oracle.OracleWeights(cfg, w)
    threads = _cpu_threads()
    n, t0 = 0, time.perf_counter()
    while n < max_frames and (n == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.run_frame(cfg, ow, inputs, n_threads=threads)
        n += 1
    dt = time.perf_counter() - t0
    n1, t1 = 0, time.perf_counter()
    while n1 < 3 and (n1 == 0 or time.perf_counter() - t1 < 5.0):
        oracle.run_frame(cfg, ow, inputs, n_threads=1, rows=[0])
        n1 += 1
    dt1 = time.perf_counter() - t1
    return {"value": n / dt, "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} whole {cfg.rows}-row frames ({dt:.1f} s) on {threads} threads",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread_us_per_frame_1row": dt1 / n1 * 1e6,
            "one_thread_sample": f"{n1} one-row frames ({dt1:.1f} s) on 1 thread"}


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


def _measured_read_rate(nbytes, reps=20):
    """Best rate of cp_stream_read (a plain HIP read kernel, 16-byte loads)
    over a working set of `nbytes`, read back to back `reps` times: GB/s."""
    import torch
    from persistent_megakernel_streaming_amd import cp
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        cp.stream_read(x, sink)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cp.stream_read(x, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del x
    torch.cuda.empty_cache()
    return nbytes / best / 1e9


CHAIN_VARIANTS = [  # (name, xcd_local, cp_chain_run variant)
    ("all_to_all_sc1_sc1", 0, 0), ("all_to_all_sys_sys", 0, 4),
    ("xcd_local_sc1_sc1", 1, 0), ("xcd_local_plain_sc1", 1, 1), ("xcd_local_plain_sc0", 1, 2),
    ("xcd_local_plain_sys", 1, 3), ("all_to_all_counter_fence", 0, 5)]


def _chain_us_per_phase(n_phases, launches=10):
    """µs per phase of empty chains of tagged-word hand-offs over 256 one-wave
    workgroups, for each store / load cache policy and scope, and of the same
    all-to-all chain handed off through a counter with release / acquire
    fences: best of `launches`; None where a wait gave up (stores its readers
    never saw)."""
    import torch
    from persistent_megakernel_streaming_amd import cp
    out = {}
    for name, local, variant in CHAIN_VARIANTS:
        slots = torch.zeros(2 * 256 * 4 + 4, dtype=torch.int32, device="cuda")  # (+ the counter of variant 5)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        base, best = 0, float("inf")
        for i in range(launches + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            cp.chain_run(slots, 256, n_phases, base, local, err, variant=variant)
            e1.record()
            torch.cuda.synchronize()
            base += n_phases
            if int(err.item()) != 0:
                break
            if i >= 2:
                best = min(best, e0.elapsed_time(e1) * 1e3)
        out[name] = None if int(err.item()) != 0 else best / n_phases
    return out


def calibrate_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": 5}), flush=True)


def _trace_frames(out_dir, wdev, steps=3):
    """Traced frames of the 5-layer loop at 64 and 1 rows, greedy, and at 64
    rows sampled: the decoded split (markdown) and the raw stamps and task
    table, written to out_dir."""
    import torch
    from persistent_megakernel_streaming_amd import cp, synth, trace
    os.makedirs(out_dir, exist_ok=True)
    res = {}
    for rows, sampled in ((64, False), (1, False), (64, True)):
        cfg = synth.CONFIGS["l5_r64_sampled" if sampled else "l5_r64"].with_(rows=rows)
        plan = cp.Plan(cfg, wdev, exec_mode="persistent", max_rows=rows, flags=cp.CP_FLAG_TRACE)
        io = cp.make_io(cfg, synth.make_inputs(cfg, sampled=sampled), logits=False)
        io["trace"] = torch.zeros(plan.info().trace_words, dtype=torch.int64, device="cuda")
        for _ in range(steps):
            plan.run(io)
        torch.cuda.synchronize()
        plan.device_status()
        table = plan.task_table()
        words = io["trace"].cpu().numpy().view(np.uint64)
        name = f"trace_l5_r{rows}" + ("_sampled" if sampled else "")
        np.savez(os.path.join(out_dir, name + ".npz"), words=words, table=table)
        s = trace.summary(trace.decode(words, table), table)
        with open(os.path.join(out_dir, name + ".md"), "w") as f:
            f.write(trace.markdown(s) + "\n")
        res[str(rows) + ("s" if sampled else "")] = s
        plan.close()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="",
                    help="comma list of p64,p1,s64,pp64,pp1,l10,floor,chain,cold,pct (default all)")
    ap.add_argument("--trace", default="", help="write traced 64- and 1-row frames to this directory and exit")
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

    everything = {"p64", "p1", "p128", "s64", "pp64", "pp1", "nolocal", "rg", "cross", "qk", "l10", "floor", "chain",
                  "cold", "pct"}
    only = set(args.only.split(",")) if args.only else everything
    steps, warm, reps = args.steps, args.warmup, args.repeats
    cfg64 = synth.CONFIGS["l5_r64"]
    w = synth.make_weights(cfg64)
    wdev = cp.upload_weights(cfg64, w)
    if args.trace:
        res = _trace_frames(args.trace, wdev)
        print(json.dumps({str(k): {kk: v[kk] for kk in ("frame_us", "handoff_us", "body_us")}
                          for k, v in res.items()}), flush=True)
        return
    res, extra = {}, {}
    plan = cp.Plan(cfg64, wdev, exec_mode="persistent", max_rows=64)
    info = plan.info()
    wbytes = info.weight_bytes_per_frame
    phases = info.n_phases
    io64 = cp.make_io(cfg64, synth.make_inputs(cfg64), logits=False)
    if "p64" in only:
        res["persistent_us_64"] = _time_frames(plan, io64, steps, warm, reps)
    if "pct" in only:
        t = _per_frame_us(plan, io64, 200)
        extra["per_frame_us_64rows"] = {"p50": float(np.percentile(t, 50)), "p99": float(np.percentile(t, 99)),
                                        "frames": len(t)}
    scrub = None
    if "cold" in only:
        scrub = torch.ones(256 * 1024 * 1024, dtype=torch.int16, device="cuda")  # 512 MiB
        t = _per_frame_us(plan, io64, 20, scrub=scrub)
        extra["cold_us_64rows"] = float(np.median(t))
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
        if "pct" in only:
            t = _per_frame_us(plan1, io1, 200)
            extra["per_frame_us_1row"] = {"p50": float(np.percentile(t, 50)), "p99": float(np.percentile(t, 99)),
                                          "frames": len(t)}
        plan1.close()
    if "p128" in only:
        # the 128-row frame (two groups of 64 rows per projection task)
        c = synth.CONFIGS["l5_r128"]
        pl = cp.Plan(c, wdev, exec_mode="persistent", max_rows=128)
        io = cp.make_io(c, synth.make_inputs(c), logits=False)
        res["persistent_us_128"] = _time_frames(pl, io, max(20, steps // 2), warm, 3)
        pl.close()
    if "qk" in only:
        # the QK-norm variant (RMSNorm of every q and k head before RoPE)
        cq = synth.CONFIGS["l5_qk_r64"]
        wq = cp.upload_weights(cq, synth.make_weights(cq))
        for mr in (64, 1):
            c = cq.with_(rows=mr)
            pl = cp.Plan(c, wq, exec_mode="persistent", max_rows=mr)
            io = cp.make_io(c, synth.make_inputs(c), logits=False)
            res[f"qk_norm_persistent_us_{mr}"] = _time_frames(pl, io, max(20, steps // 2), warm, 3)
            pl.close()
        del wq
    if "nolocal" in only:
        # every hand-off written through to memory (no XCD-local L2 hand-offs)
        for c, mr in ((cfg64, 64), (cfg1, 1)):
            pl = cp.Plan(c, wdev, exec_mode="persistent", max_rows=mr, flags=cp.CP_FLAG_NO_LOCAL)
            io = cp.make_io(c, synth.make_inputs(c), logits=False)
            res[f"write_through_persistent_us_{mr}"] = _time_frames(pl, io, max(20, steps // 2), warm, 3)
            pl.close()
    if "rg" in only:
        # two 32-row groups per projection tile, run back to back (CP_FLAG_ROW_GROUPS)
        pl = cp.Plan(cfg64, wdev, exec_mode="persistent", max_rows=64, flags=cp.CP_FLAG_ROW_GROUPS)
        io = cp.make_io(cfg64, synth.make_inputs(cfg64), logits=False)
        res["row_groups_persistent_us_64"] = _time_frames(pl, io, max(20, steps // 2), warm, 3)
        pl.close()
    if "cross" in only:
        # the row-count crossover: persistent frame against the per-phase
        # loop (captured as a graph) on one plan, rows 1 .. 64
        pl = cp.Plan(cfg64, wdev, exec_mode="persistent", max_rows=64)
        cross = {}
        for r in (1, 2, 4, 8, 16, 32, 64):
            io = cp.make_io(cfg64, synth.make_inputs(cfg64, rows=r), logits=False)
            pl.set_crossover(0)
            a = _time_frames(pl, io, 40, 5, 3)[0]
            pl.set_crossover(r + 1)
            b = _time_frames(pl, io, 40, 5, 3, graph=True)[0]
            cross[r] = {"persistent_us": a, "per_phase_graph_us": b}
        pl.set_crossover(0)
        pl.close()
        slower = [r for r, v in cross.items() if v["persistent_us"] >= v["per_phase_graph_us"]]
        extra["crossover"] = {"by_rows": cross, "rows_where_per_phase_wins": slower}
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
    l10_bytes = None
    if "l10" in only:
        cfg10 = synth.CONFIGS["l10_r64"]
        w10 = cp.upload_weights(cfg10, synth.make_weights(cfg10))
        for rows in (1, 16, 64):
            c = cfg10.with_(rows=rows)
            pl = cp.Plan(c, w10, exec_mode="persistent", max_rows=rows)
            io = cp.make_io(c, synth.make_inputs(c), logits=False)
            res[f"l10_persistent_us_{rows}"] = _time_frames(pl, io, max(20, steps // 4), warm, 3)
            l10_bytes = pl.info().weight_bytes_per_frame
            if rows == 64 and scrub is not None:
                extra["l10_cold_us_64rows"] = float(np.median(_per_frame_us(pl, io, 20, scrub=scrub)))
            pl.close()
        del w10
        torch.cuda.empty_cache()
    del scrub
    floor = None
    if "floor" in only:
        g157 = _measured_read_rate(157 * 1000 * 1000)
        g314 = _measured_read_rate(314 * 1000 * 1000)
        floor = {"read_GBps_157MB": g157, "read_GBps_314MB": g314,
                 "measured_floor_us_5layers": wbytes / (g157 * 1e3),
                 "measured_floor_us_10layers": (l10_bytes / (g314 * 1e3)) if l10_bytes else None,
                 "kernel": "cp_stream_read (plain HIP read, 16-byte loads, 4096 x 256 threads)"}
    if "chain" in only:
        ch = _chain_us_per_phase(phases)
        a2a = ch["all_to_all_sc1_sc1"]
        extra["empty_chain"] = {"us_per_phase": ch, "phases": phases,
                                "chain_bound_us_all_to_all": a2a * phases if a2a else None}

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
        "vs_baseline": None,
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
        "gap_to_2x_floor_us_64rows": (us64 - 2 * floor_us) if us64 else None,
        "h200_context_us": {"persistent_1row": 2127.0, "persistent_64rows": H200_US_64ROWS,
                            "frame_in_59row_step": 2220.0, "floor_at_4.8TBps": 537.8},
        "measured_floor": floor,
        "detail_us_median_min_max": res,
        "repeats": reps,
    }
    out.update(extra)
    if us64:
        achieved = wbytes / (us64 * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS, "traffic": _stored_traffic(),
                           "traffic_counts": "FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated: bytes between "
                                             "the L2s and the memory side (Infinity Cache or HBM)"}
    if us1:
        a1 = wbytes / (us1 * 1e-6) / 1e9
        out["roofline_1row"] = {"bound": "hbm", "achieved": a1, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": a1 / HBM_PEAK_GBPS}
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(cfg64, w, synth.make_inputs(cfg64))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
