"""Decoder of the persistent executor's per-task timestamps (reporting only).

A frame run with ``CP_FLAG_TRACE`` and a trace buffer writes eight
timestamps per task (include/cp.h, ``cp_frame_io.trace``); the task table
(``cp_plan_task_table``) says which phase, kind and workgroup each task is.
This module turns the two into the per-phase split of the mstar pull request
"Qwen3-TTS: Run the 1.7B Depth Loop as One Persistent Kernel on Hopper",
section "Where the depth loop's time goes" (bullet "Phases": time in the
hand-offs between phases against time in each phase's slowest task; bullet
"Inside a task": where a task's time goes).

For every phase k let E_k be the latest "outputs issued" stamp of its tasks
and c_k the task that issued it.  Then
  * hand-off_k = (c_k's "dependencies met" stamp) - E_{k-1}: from the previous
    phase's last output to the moment the task that ends this phase had its
    inputs (negative when that task did not wait for the previous phase's
    last task);
  * body_k = E_k - (c_k's "dependencies met" stamp).
The two sum, over the frame, to E_last - E_first.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01  # s_memrealtime counts a 100 MHz clock

KINDS = {1: "inproj", 2: "embed0", 3: "qkv", 4: "attn", 5: "o", 6: "gate/up", 7: "down", 8: "head", 9: "draw"}
PROJ = (1, 3, 5, 6, 7, 8)
# stamp indices (include/cp.h)
S_START, S_DISPATCH, S_DEPS, S_GROUP0, S_KLOOP, S_OUT, S_BARRIER, S_ISSUE = range(8)


def decode(trace_words, table):
    """Per-task stamps in microseconds from the frame's earliest start.

    ``trace_words``: the frame's trace (uint64, n_tasks * 8); ``table``: the
    plan's task table ([n_tasks][8] int32).  Stamps a task did not write this
    frame (outside its own start .. issue span, or kinds that do not pass
    through them) are NaN."""
    t = np.asarray(trace_words, dtype=np.uint64).reshape(-1, 8).astype(np.int64)
    tab = np.asarray(table)
    kind = tab[:, 1]
    t0 = t[:, S_START].min()
    us = (t - t0).astype(np.float64) * TICK_US
    lo, hi = us[:, S_START:S_START + 1], us[:, S_ISSUE:S_ISSUE + 1]
    us[(us < lo) | (us > hi)] = np.nan
    has_deps = np.isin(kind, PROJ + (4, 9))
    us[~has_deps, S_DEPS] = np.nan
    us[~np.isin(kind, PROJ), S_GROUP0:S_KLOOP + 1] = np.nan
    return us


def check_monotone(us, table):
    """Problems with the stamps' order (empty list if none): within a task the
    stamps it wrote rise; along a workgroup's list each task starts after the
    previous one issued its next tile copy."""
    bad = []
    order = [S_START, S_DISPATCH, S_DEPS, S_GROUP0, S_KLOOP, S_OUT, S_BARRIER, S_ISSUE]
    for i, row in enumerate(us):
        v = [row[k] for k in order if not np.isnan(row[k])]
        if any(b < a for a, b in zip(v, v[1:])):
            bad.append(("task", i, row.tolist()))
    tab = np.asarray(table)
    for w in np.unique(tab[:, 6]):
        idx = np.where(tab[:, 6] == w)[0]
        idx = idx[np.argsort(tab[idx, 7])]
        for a, b in zip(idx, idx[1:]):
            if us[b, S_START] < us[a, S_ISSUE]:
                bad.append(("workgroup", int(w), int(a), int(b)))
    return bad


def phase_split(us, table):
    """Per phase: (phase, kind, layer, position, hand-off µs, body µs, end µs)."""
    tab = np.asarray(table)
    phases = np.unique(tab[:, 0])
    rows = []
    prev_end = None
    for ph in phases:
        idx = np.where(tab[:, 0] == ph)[0]
        out = us[idx, S_OUT]
        c = idx[int(np.nanargmax(out))]
        end = us[c, S_OUT]
        deps = us[c, S_DEPS] if not np.isnan(us[c, S_DEPS]) else us[c, S_DISPATCH]
        hand = (deps - prev_end) if prev_end is not None else 0.0
        rows.append((int(ph), int(tab[c, 1]), int(tab[c, 2]), int(tab[c, 3]), float(hand), float(end - deps),
                     float(end)))
        prev_end = end
    return rows


def summary(us, table):
    """Totals by phase kind and medians of each task interval by task kind."""
    tab = np.asarray(table)
    split = phase_split(us, table)
    by_kind = {}
    for _, k, _, _, hand, body, _ in split:
        d = by_kind.setdefault(KINDS[k], [0, 0.0, 0.0])
        d[0] += 1
        d[1] += hand
        d[2] += body
    intervals = {"dispatch": (S_START, S_DISPATCH), "wait": (S_DISPATCH, S_DEPS), "group0": (S_DEPS, S_GROUP0),
                 "kloop": (S_GROUP0, S_KLOOP), "epilogue": (S_KLOOP, S_OUT), "body": (S_DEPS, S_OUT),
                 "barrier": (S_OUT, S_BARRIER), "issue": (S_BARRIER, S_ISSUE)}
    med = {}
    for k, name in KINDS.items():
        idx = np.where(tab[:, 1] == k)[0]
        if len(idx) == 0:
            continue
        med[name] = {}
        for iname, (a, b) in intervals.items():
            d = us[idx, b] - us[idx, a]
            d = d[~np.isnan(d)]
            med[name][iname] = float(np.median(d)) if len(d) else None
    frame = split[-1][6] - float(np.nanmin(us[:, S_START]))
    return {"frame_us": frame, "n_phases": len(split),
            "handoff_us": sum(r[4] for r in split), "body_us": sum(r[5] for r in split),
            "by_phase_kind": {k: {"phases": v[0], "handoff_us": v[1], "body_us": v[2]} for k, v in by_kind.items()},
            "task_median_us": med}


def markdown(s):
    """The summary as two markdown tables."""
    out = [f"Frame span {s['frame_us']:.1f} us over {s['n_phases']} phases: "
           f"hand-offs {s['handoff_us']:.1f} us, phase bodies {s['body_us']:.1f} us.", "",
           "| phase kind | phases | hand-off us (sum) | body us (sum) | hand-off us / phase | body us / phase |",
           "|---|---|---|---|---|---|"]
    for k, v in s["by_phase_kind"].items():
        n = v["phases"]
        out.append(f"| {k} | {n} | {v['handoff_us']:.1f} | {v['body_us']:.1f} | {v['handoff_us'] / n:.2f} | "
                   f"{v['body_us'] / n:.2f} |")
    cols = ["dispatch", "wait", "group0", "kloop", "epilogue", "body", "barrier", "issue"]
    out += ["", "Median per task (us):", "", "| task kind | " + " | ".join(cols) + " |",
            "|---|" + "---|" * len(cols)]
    for k, v in s["task_median_us"].items():
        out.append(f"| {k} | " + " | ".join("-" if v[c] is None else f"{v[c]:.2f}" for c in cols) + " |")
    return "\n".join(out)
