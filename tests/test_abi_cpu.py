"""Host-only checks of the C ABI library: it loads, exports every function
include/cp.h declares, rejects bad arguments before touching a device, and its
planner builds deadlock-free task lists (no GPU needed)."""
import ctypes as C

import numpy as np
import os
import re

import pytest

from persistent_megakernel_streaming_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cp():
    from persistent_megakernel_streaming_amd import cp
    return cp


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "cp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    cp = _cp()
    names = _declared_functions()
    assert "cp_plan_create" in names and "cp_frame_run" in names and "cp_plan_destroy" in names
    for n in names:
        assert hasattr(cp.lib(), n), n


def test_status_strings_and_null_arguments():
    cp = _cp()
    lib = cp.lib()
    for s in range(7):
        assert lib.cp_status_string(s)
    assert lib.cp_plan_create(None, None, 0, None) == 1
    h = C.c_void_p()
    c = cp.make_config(synth.CONFIGS["tiny_f32"])
    assert lib.cp_plan_create(C.byref(c), None, 0, C.byref(h)) == 1 and not h.value
    assert lib.cp_plan_destroy(None) == 0
    assert lib.cp_frame_run(None, None, None) == 1
    assert lib.cp_plan_set_epoch(None, 1) == 1


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=96), 2), (dict(n_positions=17), 2), (dict(n_kv_heads=3), 2),
    (dict(hidden=1000), 2), (dict(n_layers=0), 1), (dict(rows=129), 2),
])
def test_unsupported_shapes_are_refused_on_the_host(change, status):
    cp = _cp()
    rows = change.pop("rows", None)
    cfg = synth.CONFIGS["l5_r1"].with_(**change)
    c = cp.make_config(cfg, max_rows=rows)
    info = cp.PlanInfo()
    assert cp.lib().cp_schedule_check(C.byref(c), 256, C.byref(info)) == status
    assert cp.lib().cp_last_create_error()


@pytest.mark.parametrize("name", ["tiny_f32", "l5_r1", "l5_r64", "l10_r64", "l5_in2048_r8", "l5_qk_r64", "l5_r128"])
@pytest.mark.parametrize("cus", [256, 64, 7])
def test_schedule_invariants(name, cus):
    cp = _cp()
    cfg = synth.CONFIGS[name]
    info = cp.schedule_check(cfg, cu_count=cus)
    L, P = cfg.n_layers, cfg.n_positions
    # 5 L P + 2 P phases (input projection, 15 heads, 16 embedding steps), less
    # the four phases after position 0's last qkv, whose results nothing reads
    # (three with QK-norm, whose attention there writes the normed K).
    assert info.n_phases == 5 * L * P + 2 * P - (3 if cfg.qk_norm else 4)
    assert info.n_workgroups == cus
    assert info.max_tasks_per_workgroup * cus >= info.n_tasks


@pytest.mark.parametrize("name", ["l5_r64", "l5_r128", "l5_qk_r64", "l5_in2048_r8", "l5_r1"])
@pytest.mark.parametrize("cus", [256, 64, 7])
def test_row_group_schedule_invariants(name, cus):
    """CP_FLAG_ROW_GROUPS: every projection task of a plan of more than 32
    rows becomes one task per 32-row group on the same workgroup (the
    schedule check accepts the lists); plans of at most 32 rows are unchanged."""
    cp = _cp()
    cfg = synth.CONFIGS[name]
    a = cp.schedule_check(cfg, cu_count=cus)
    b = cp.schedule_check(cfg, cu_count=cus, flags=cp.CP_FLAG_ROW_GROUPS)
    assert b.n_phases == a.n_phases
    if cfg.rows <= 32:
        assert b.n_tasks == a.n_tasks
    else:
        assert b.n_tasks > a.n_tasks
    c = cp.make_config(cfg, exec_mode="per_phase", flags=cp.CP_FLAG_ROW_GROUPS)
    info = cp.PlanInfo()
    assert cp.lib().cp_schedule_check(C.byref(c), cus, C.byref(info)) == 2  # persistent executor only


def test_head_and_one_row_gate_up_tiles_avoid_the_split_k_owners():
    """The head tiles of each position go to workgroups other than the last
    down phase's split-K owners (at 256 CUs there are enough of them), and in
    a one-row plan the gate/up tiles go to workgroups other than the o
    owners; 64-row gate/up keeps its plain rotation."""
    cp = _cp()
    T_O, T_GU, T_DOWN, T_HEAD = 5, 6, 7, 8
    for name in ("l5_r1", "l5_r64"):
        cfg = synth.CONFIGS[name]
        tab = cp.schedule_task_table(cfg, cu_count=256)
        ph, ty, lay, pos, split, wg = tab[:, 0], tab[:, 1], tab[:, 2], tab[:, 3], tab[:, 5], tab[:, 6]
        for p in range(1, cfg.n_positions):
            owners = set(wg[(ty == T_DOWN) & (lay == cfg.n_layers - 1) & (pos == p) & (split == 0)].tolist())
            heads = set(wg[(ty == T_HEAD) & (pos == p)].tolist())
            assert heads and not heads & owners, (name, p)
        clash = 0
        for p in range(1, cfg.n_positions):
            for l in range(cfg.n_layers):
                owners = set(wg[(ty == T_O) & (lay == l) & (pos == p) & (split == 0)].tolist())
                gu = set(wg[(ty == T_GU) & (lay == l) & (pos == p)].tolist())
                clash += len(gu & owners)
        if cfg.rows == 1:
            assert clash == 0
        else:
            assert clash > 0  # plain rotation at 64 rows


def test_schedule_task_table_matches_the_schedule_check():
    cp = _cp()
    cfg = synth.CONFIGS["tiny_f32"]
    info = cp.schedule_check(cfg, cu_count=7)
    tab = cp.schedule_task_table(cfg, cu_count=7)
    assert tab.shape == (info.n_tasks, 8)
    assert len(np.unique(tab[:, 0])) == info.n_phases
    assert tab[:, 6].max() == 6
    for w in range(7):  # each workgroup's list is in phase order, indexed 0..n-1
        mine = tab[tab[:, 6] == w]
        assert np.array_equal(mine[:, 7], np.arange(len(mine)))
        assert np.all(np.diff(mine[:, 0]) >= 0)
    c = cp.make_config(cfg)
    out = np.zeros((info.n_tasks + 1, 8), np.int32)
    assert cp.lib().cp_schedule_task_table(C.byref(c), 7, out.ctypes.data, info.n_tasks + 1) == 1


def test_qk_norm_gains_are_plan_constants():
    """The QK-norm variant keeps its head-norm gains ([L][q, k][head_dim]
    fp32) with the plan's constants; the schedule gains one phase, position
    0's last-layer attention, which writes that position's normed K."""
    cp = _cp()
    base, qk = synth.CONFIGS["l5_r64"], synth.CONFIGS["l5_qk_r64"]
    a, b = cp.schedule_check(base), cp.schedule_check(qk)
    assert b.const_bytes - a.const_bytes == -(-(qk.n_layers * 2 * qk.head_dim * 4) // 256) * 256
    assert b.n_phases == a.n_phases + 1
    assert b.n_tasks == a.n_tasks + qk.n_kv_heads * 32  # 64 rows: 32 two-row attention tasks per kv head


def test_inline_asm_vector_memory_blocks_start_with_the_guard(tmp_path):
    """Every inline-asm block that issues a vector-memory instruction starts
    with five wait states (the build refuses the source otherwise): the
    compiler does not guard asm against reading SGPRs a VALU instruction has
    just written, and an unguarded block faulted the GPU."""
    from persistent_megakernel_streaming_amd import build
    src = os.path.join(ROOT, "persistent_megakernel_streaming_amd", "csrc", "cp_kernels.hip")
    assert build.check_asm_guards(src) >= 8
    bad = tmp_path / "bad.hip"
    bad.write_text('asm volatile("s_nop 4\\n"\n "s_waitcnt vmcnt(0)" ::: "memory");\n'
                   'asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen sc1\\n"\n'
                   '             "s_waitcnt vmcnt(0)" : "+v"(v) : "v"(o), "s"(r) : "memory");\n')
    with pytest.raises(RuntimeError, match="bad.hip:3"):
        build.check_asm_guards(str(bad))
    bad.write_text('asm volatile("s_nop 1\\nglobal_store_dword %0, %1, off" :: "v"(a), "v"(b));\n')
    with pytest.raises(RuntimeError):
        build.check_asm_guards(str(bad))
    # a load's outputs must not be able to share the address's registers
    bad.write_text('asm volatile("s_nop 4\\ns_load_dwordx4 %0, %2, 0x0\\ns_load_dwordx2 %1, %2, 0x10"\n'
                   '             : "=s"(a), "=&s"(b) : "s"(t));\n')
    with pytest.raises(RuntimeError, match="early-clobber"):
        build.check_asm_guards(str(bad))
    bad.write_text('asm volatile("s_nop 4\\ns_load_dwordx4 %0, %2, 0x0\\ns_load_dwordx2 %1, %2, 0x10"\n'
                   '             : "=&s"(a), "=&s"(b) : "s"(t));\n')
    assert build.check_asm_guards(str(bad)) == 1


@pytest.mark.parametrize("args", [
    (256, 8, 0, 1, 5),        # the counter form is all-to-all only
    (256, 8, 0, 0, 6),        # no such variant
    (256, 8, 0, 0, 1),        # plain stores need the XCD-local chain
    (256, 8, (1 << 24) - 8, 0, 5),  # the counter would pass 2^32
    (0, 8, 0, 0, 0),          # no workgroups
])
def test_chain_probe_refusals(args):
    """cp_chain_run refuses, before any launch, a variant it does not have or
    a combination the hand-off it measures cannot run (no device needed)."""
    from persistent_megakernel_streaming_amd import cp
    n_wg, n_ph, base, local, variant = args
    lib = cp.lib()
    st = lib.cp_chain_run(C.c_void_p(16), n_wg, n_ph, base, local, variant, C.c_void_p(16), None)
    assert st == cp.CP_ERR_INVALID_ARGUMENT
