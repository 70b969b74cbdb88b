"""The allocation-free plan (cp_plan_create_static) against cp_plan_create.

A static plan takes its scratch from the array the library holds on each
device and its constants from a caller's arena; its frames run the same
kernels, so they must equal an allocating plan's frames bit for bit.  Two
plans in a row (the second with a smaller frame, on a smaller plan) share
the array: the second must not see anything the first left in it.
"""
import numpy as np
import pytest
import torch

from persistent_megakernel_streaming_amd import synth

pytestmark = pytest.mark.gpu


def _cp():
    from persistent_megakernel_streaming_amd import cp
    return cp


def _frame(plan, cfg, inputs):
    cp = _cp()
    io = cp.make_io(cfg, inputs, kv=True)
    plan.run(io)
    torch.cuda.synchronize()
    plan.device_status()
    return {k: v.cpu().numpy() for k, v in io.items() if k != "rows"}


def test_static_plan_equals_allocating_plan_twice():
    cp = _cp()
    cfg = synth.CONFIGS["l5_r64"]
    wdev = cp.upload_weights(cfg, synth.make_weights(cfg))
    arena = torch.empty(cp.schedule_check(cfg, max_rows=64).const_bytes, dtype=torch.uint8, device="cuda")
    for rows, max_rows in ((64, 64), (13, 16)):
        c = cfg.with_(rows=rows)
        inputs = synth.make_inputs(c, seed=rows)
        ref_plan = cp.Plan(c, wdev, max_rows=max_rows)
        ref = _frame(ref_plan, c, inputs)
        ref_plan.close()
        st = cp.Plan(c, wdev, max_rows=max_rows, weight_arena=arena)
        got = [_frame(st, c, inputs) for _ in range(2)]  # two frames on the static plan
        st.close()
        for i, g in enumerate(got):
            for k in ref:
                assert np.array_equal(ref[k], g[k]), (rows, i, k)


def test_static_plan_refusals():
    """One live static plan per device; an arena below const_bytes and a plan
    whose scratch exceeds the array are refused on the host with a message."""
    cp = _cp()
    cfg = synth.CONFIGS["tiny_f32"].with_(rows=2, dtype="bf16")
    wdev = cp.upload_weights(cfg, synth.make_weights(cfg, seed=3))
    need = cp.schedule_check(cfg, max_rows=2).const_bytes
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(cp.CpError) as e:
        cp.Plan(cfg, wdev, max_rows=2, weight_arena=small)
    assert e.value.status == cp.CP_ERR_INVALID_ARGUMENT and "arena" in str(e.value)
    arena = torch.empty(need, dtype=torch.uint8, device="cuda")
    a = cp.Plan(cfg, wdev, max_rows=2, weight_arena=arena)
    arena2 = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(cp.CpError) as e:
        cp.Plan(cfg, wdev, max_rows=2, weight_arena=arena2)
    assert e.value.status == cp.CP_ERR_INVALID_ARGUMENT and "already" in str(e.value)
    inputs = synth.make_inputs(cfg, seed=3)
    ref_plan = cp.Plan(cfg, wdev, max_rows=2)
    ref = _frame(ref_plan, cfg, inputs)
    ref_plan.close()
    got = _frame(a, cfg, inputs)
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k
    a.close()
    big = synth.CONFIGS["l10_r64"]
    w10 = cp.upload_weights(big, synth.make_weights(big))
    arena10 = torch.empty(cp.schedule_check(big, max_rows=64).const_bytes, dtype=torch.uint8, device="cuda")
    with pytest.raises(cp.CpError) as e:
        cp.Plan(big, w10, max_rows=64, weight_arena=arena10)
    assert e.value.status == cp.CP_ERR_OUT_OF_MEMORY and "bytes" in str(e.value)
    # the refusals left no live static plan behind
    b = cp.Plan(cfg, wdev, max_rows=2, weight_arena=arena)
    b.close()
