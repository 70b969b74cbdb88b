"""Host checks of the trace decoder (persistent_megakernel_streaming_amd.trace)
on a synthetic task table and trace whose split is known by construction."""
import numpy as np

from persistent_megakernel_streaming_amd import trace


def _synthetic():
    """Three phases on two workgroups: phase 0 (qkv) tasks end at 10 and 12;
    phase 1 (attention) task waits until 15 and ends at 20; phase 2 (o) tasks
    get their inputs at 23 and 24 and end at 30 and 27.  Times in 10 ns ticks
    of the device clock, offset by a base."""
    base = 1_000_000
    # phase, type, layer, pos, tile, split, workgroup, index in workgroup
    table = np.array([[0, 3, 0, 0, 0, 0, 0, 0], [0, 3, 0, 0, 1, 0, 1, 0],
                      [1, 4, 0, 0, 0, 0, 0, 1],
                      [2, 5, 0, 0, 0, 0, 0, 2], [2, 5, 0, 0, 0, 1, 1, 1]], np.int32)
    t = np.array([
        [0, 1, 2, 3, 4, 10, 11, 11],
        [0, 1, 3, 4, 5, 12, 12, 13],
        [11, 12, 15, 0, 0, 20, 21, 21],
        [21, 21, 23, 25, 28, 30, 30, 31],
        [13, 14, 24, 25, 26, 27, 28, 29],
    ], np.int64) * 100 + base
    t[2, 3:5] = 5  # attention does not pass through the K-loop stamps (stale words)
    return table, t.astype(np.uint64).reshape(-1)


def test_decode_split_and_order():
    table, words = _synthetic()
    us = trace.decode(words, table)
    assert np.isnan(us[2, trace.S_GROUP0]) and np.isnan(us[2, trace.S_KLOOP])
    assert us[0, trace.S_START] == 0.0 and us[3, trace.S_OUT] == 30.0
    assert trace.check_monotone(us, table) == []
    split = trace.phase_split(us, table)
    # phase 0 ends at 12 (task 1, inputs at 3); phase 1 at 20 (inputs at 15);
    # phase 2 at 30 (task 3, inputs at 23)
    assert [(r[4], r[5], r[6]) for r in split] == [(0.0, 9.0, 12.0), (3.0, 5.0, 20.0), (3.0, 7.0, 30.0)]
    s = trace.summary(us, table)
    # hand-offs and bodies add up to the span from the first phase's input to the last output
    assert abs(s["handoff_us"] + s["body_us"] - (30.0 - 3.0)) < 1e-9
    assert s["frame_us"] == 30.0
    assert s["by_phase_kind"]["o"] == {"phases": 1, "handoff_us": 3.0, "body_us": 7.0}
    assert s["task_median_us"]["qkv"]["body"] == (8.0 + 9.0) / 2
    assert "| o | 1 |" in trace.markdown(s)


def test_monotone_check_finds_disorder():
    table, words = _synthetic()
    t = words.reshape(-1, 8).copy()
    t[4, trace.S_START] = t[1, trace.S_ISSUE] - 100  # starts before its workgroup's previous task issued
    us = trace.decode(t.reshape(-1), table)
    bad = trace.check_monotone(us, table)
    assert bad and bad[0][0] == "workgroup"
