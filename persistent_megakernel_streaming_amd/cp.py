"""Thin ctypes binding of libcpms.so (include/cp.h).

Argument marshalling only: every step of the depth loop runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is not built, importing this module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcpms.so")

CP_OK = 0
STATUS = {0: "CP_OK", 1: "CP_ERR_INVALID_ARGUMENT", 2: "CP_ERR_UNSUPPORTED", 3: "CP_ERR_NOT_CORESIDENT",
          4: "CP_ERR_OUT_OF_MEMORY", 5: "CP_ERR_HIP", 6: "CP_ERR_DEVICE_TIMEOUT"}
(CP_ERR_INVALID_ARGUMENT, CP_ERR_UNSUPPORTED, CP_ERR_NOT_CORESIDENT, CP_ERR_OUT_OF_MEMORY, CP_ERR_HIP,
 CP_ERR_DEVICE_TIMEOUT) = range(1, 7)
CP_DTYPE_F32, CP_DTYPE_BF16 = 0, 1
CP_EXEC_PERSISTENT, CP_EXEC_PER_PHASE = 0, 1
CP_FLAG_TRACE = 1
CP_FLAG_NO_LOCAL = 4
CP_FLAG_ROW_GROUPS = 8
ABI_VERSION = 3
EPOCH_WRAP = (1 << 22) - 1  # epochs run 1 .. EPOCH_WRAP - 1

_VP = C.c_void_p


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("abi_version", "n_layers", "hidden", "input_dim", "n_q_heads",
                                          "n_kv_heads", "head_dim", "intermediate", "n_positions", "vocab",
                                          "max_rows", "dtype")] + [
        ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("exec", C.c_int32), ("flags", C.c_uint32),
        ("qk_norm", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [("w_in", _VP), ("embed", C.POINTER(_VP)), ("attn_norm", C.POINTER(_VP)),
                ("w_qkv", C.POINTER(_VP)), ("w_o", C.POINTER(_VP)), ("mlp_norm", C.POINTER(_VP)),
                ("w_gate", C.POINTER(_VP)), ("w_up", C.POINTER(_VP)), ("w_down", C.POINTER(_VP)),
                ("final_norm", _VP), ("w_head", C.POINTER(_VP)), ("q_norm", C.POINTER(_VP)),
                ("k_norm", C.POINTER(_VP))]


class FrameIO(C.Structure):
    _fields_ = [("rows", C.c_int32), ("hidden_in", _VP), ("code0", _VP), ("temperature", _VP),
                ("top_k", _VP), ("top_p", _VP), ("seed", _VP), ("offset", _VP), ("codes", _VP),
                ("embsum", _VP), ("logits", _VP), ("k_cache", _VP), ("v_cache", _VP), ("trace", _VP)]


class PlanInfo(C.Structure):
    _fields_ = [("n_phases", C.c_int32), ("n_tasks", C.c_int32), ("n_workgroups", C.c_int32),
                ("lds_bytes", C.c_int32), ("weight_bytes_per_frame", C.c_int64),
                ("packed_weight_bytes", C.c_int64), ("scratch_bytes", C.c_int64), ("trace_words", C.c_int64),
                ("cu_count", C.c_int32), ("max_tasks_per_workgroup", C.c_int32), ("const_bytes", C.c_int64)]


class CpError(RuntimeError):
    def __init__(self, status, msg=""):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run persistent_megakernel_streaming_amd.build")
    lib = C.CDLL(LIB_PATH)
    lib.cp_plan_create.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.c_int, C.POINTER(C.c_void_p)]
    lib.cp_plan_create_static.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.c_int, C.c_void_p, C.c_uint64,
                                          C.POINTER(C.c_void_p)]
    lib.cp_frame_run.argtypes = [C.c_void_p, C.POINTER(FrameIO), C.c_void_p]
    lib.cp_plan_destroy.argtypes = [C.c_void_p]
    lib.cp_plan_query.argtypes = [C.c_void_p, C.POINTER(PlanInfo)]
    lib.cp_plan_device_status.argtypes = [C.c_void_p]
    lib.cp_status_string.argtypes = [C.c_int]
    lib.cp_status_string.restype = C.c_char_p
    lib.cp_plan_last_error.argtypes = [C.c_void_p]
    lib.cp_plan_last_error.restype = C.c_char_p
    lib.cp_last_create_error.restype = C.c_char_p
    lib.cp_schedule_check.argtypes = [C.POINTER(Config), C.c_int, C.POINTER(PlanInfo)]
    lib.cp_schedule_task_table.argtypes = [C.POINTER(Config), C.c_int, C.c_void_p, C.c_int64]
    lib.cp_plan_task_table.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
    lib.cp_plan_set_epoch.argtypes = [C.c_void_p, C.c_uint32]
    lib.cp_plan_set_spin_limit.argtypes = [C.c_void_p, C.c_uint32]
    lib.cp_plan_set_crossover.argtypes = [C.c_void_p, C.c_int]
    lib.cp_stream_read.argtypes = [C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p]
    lib.cp_chain_run.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_uint32, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    for f in ("cp_plan_create", "cp_plan_create_static", "cp_frame_run", "cp_plan_destroy", "cp_plan_query", "cp_plan_device_status",
              "cp_schedule_check", "cp_schedule_task_table", "cp_plan_task_table", "cp_plan_set_epoch", "cp_plan_set_spin_limit",
              "cp_plan_set_crossover", "cp_stream_read", "cp_chain_run"):
        getattr(lib, f).restype = C.c_int
    return lib


_lib = load_library()


def lib():
    return _lib


def make_config(cfg, max_rows=None, exec_mode="persistent", flags=0) -> Config:
    """A cp_config for a synth.DepthLoopConfig-like object."""
    return Config(abi_version=ABI_VERSION, n_layers=cfg.n_layers, hidden=cfg.hidden, input_dim=cfg.input_dim,
                  n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                  intermediate=cfg.intermediate, n_positions=cfg.n_positions, vocab=cfg.vocab,
                  max_rows=cfg.rows if max_rows is None else max_rows,
                  dtype=CP_DTYPE_BF16 if cfg.dtype == "bf16" else CP_DTYPE_F32,
                  rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
                  exec=CP_EXEC_PER_PHASE if exec_mode == "per_phase" else CP_EXEC_PERSISTENT, flags=flags,
                  qk_norm=1 if getattr(cfg, "qk_norm", False) else 0)


def schedule_check(cfg, cu_count=256, max_rows=None, flags=0):
    """Builds and checks the task lists for a device of cu_count CUs (host only)."""
    c = make_config(cfg, max_rows=max_rows, flags=flags)
    info = PlanInfo()
    st = _lib.cp_schedule_check(C.byref(c), int(cu_count), C.byref(info))
    if st != CP_OK:
        raise CpError(st, _lib.cp_last_create_error().decode())
    return info


def schedule_task_table(cfg, cu_count=256, max_rows=None, flags=0) -> np.ndarray:
    """[n_tasks][8] int32 task table of the host-built schedule (phase, type,
    layer, pos, tile, split, workgroup, index in list); touches no device."""
    c = make_config(cfg, max_rows=max_rows, flags=flags)
    info = schedule_check(cfg, cu_count=cu_count, max_rows=max_rows, flags=flags)
    out = np.zeros((info.n_tasks, 8), np.int32)
    st = _lib.cp_schedule_task_table(C.byref(c), int(cu_count), out.ctypes.data, info.n_tasks)
    if st != CP_OK:
        raise CpError(st, _lib.cp_last_create_error().decode())
    return out


def _stream(stream):
    import torch
    return torch.cuda.current_stream().cuda_stream if stream is None else stream


def stream_read(buf, sink, stream=None):
    """Enqueues one plain read of device tensor ``buf`` (cp_stream_read)."""
    st = _lib.cp_stream_read(C.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                             C.c_void_p(sink.data_ptr()), C.c_void_p(_stream(stream)))
    if st != CP_OK:
        raise CpError(st, "cp_stream_read")


def chain_run(slots, n_workgroups, n_phases, tag_base, xcd_local, error_word, variant=0, stream=None):
    """Enqueues an empty chain of tagged-word hand-offs (cp_chain_run)."""
    st = _lib.cp_chain_run(C.c_void_p(slots.data_ptr()), int(n_workgroups), int(n_phases), int(tag_base),
                           int(bool(xcd_local)), int(variant), C.c_void_p(error_word.data_ptr()),
                           C.c_void_p(_stream(stream)))
    if st != CP_OK:
        raise CpError(st, "cp_chain_run")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def upload_weights(cfg, w: dict, device="cuda"):
    """Copies stored weights (numpy, storage type; bf16 as uint16 bits) to the device."""
    import torch
    out = {}
    for k, v in w.items():
        a = np.ascontiguousarray(v)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        out[k] = torch.from_numpy(a).to(device)
    return out


class Plan:
    """A cp_plan.  ``weights``: device tensors keyed as synth.make_weights names them."""

    def __init__(self, cfg, weights: dict, exec_mode="persistent", max_rows=None, device=0, flags=0,
                 weight_arena=None):
        """``weight_arena``: a device tensor of at least ``const_bytes``
        bytes makes a static plan (cp_plan_create_static: no device
        allocation; its scratch lives in the library's per-device array)."""
        self.cfg = cfg
        self._c = make_config(cfg, max_rows=max_rows, exec_mode=exec_mode, flags=flags)
        L, P = cfg.n_layers, cfg.n_positions

        def arr(names):
            a = (C.c_void_p * len(names))(*[weights[n].data_ptr() for n in names])
            return C.cast(a, C.POINTER(C.c_void_p)), a

        keep = []
        fields = {}
        for key, names in (("embed", [f"embed.{j}" for j in range(P)]),
                           ("attn_norm", [f"attn_norm.{l}" for l in range(L)]),
                           ("w_qkv", [f"w_qkv.{l}" for l in range(L)]),
                           ("w_o", [f"w_o.{l}" for l in range(L)]),
                           ("mlp_norm", [f"mlp_norm.{l}" for l in range(L)]),
                           ("w_gate", [f"w_gate.{l}" for l in range(L)]),
                           ("w_up", [f"w_up.{l}" for l in range(L)]),
                           ("w_down", [f"w_down.{l}" for l in range(L)]),
                           ("w_head", [f"w_head.{j}" for j in range(1, P)])):
            fields[key], a = arr(names)
            keep.append(a)
        if getattr(cfg, "qk_norm", False):
            for key in ("q_norm", "k_norm"):
                fields[key], a = arr([f"{key}.{l}" for l in range(L)])
                keep.append(a)
        self._w = Weights(w_in=weights["w_in"].data_ptr(), final_norm=weights["final_norm"].data_ptr(), **fields)
        h = C.c_void_p()
        if weight_arena is None:
            st = _lib.cp_plan_create(C.byref(self._c), C.byref(self._w), int(device), C.byref(h))
        else:
            st = _lib.cp_plan_create_static(C.byref(self._c), C.byref(self._w), int(device),
                                            C.c_void_p(weight_arena.data_ptr()),
                                            weight_arena.numel() * weight_arena.element_size(), C.byref(h))
        if st != CP_OK:
            raise CpError(st, _lib.cp_last_create_error().decode())
        self._h = h
        self._keep = keep

    def info(self) -> PlanInfo:
        i = PlanInfo()
        self._check(_lib.cp_plan_query(self._h, C.byref(i)))
        return i

    def last_error(self) -> str:
        """Text of the last error or note recorded on the plan ("" if none)."""
        return _lib.cp_plan_last_error(self._h).decode()

    def _check(self, st):
        if st != CP_OK:
            raise CpError(st, _lib.cp_plan_last_error(self._h).decode())

    def run(self, io: dict, stream=None):
        """Enqueues one frame.  ``io`` maps cp_frame_io field names to device
        tensors (``rows`` to an int); the call does not wait."""
        import torch
        f = FrameIO(rows=int(io["rows"]))
        for k in ("hidden_in", "code0", "temperature", "top_k", "top_p", "seed", "offset", "codes", "embsum",
                  "logits", "k_cache", "v_cache", "trace"):
            t = io.get(k)
            if t is not None:
                setattr(f, k, t.data_ptr())
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        self._check(_lib.cp_frame_run(self._h, C.byref(f), C.c_void_p(s)))

    def task_table(self) -> np.ndarray:
        """[n_tasks][8] int32: phase, type, layer, pos, tile, split, workgroup, index in list."""
        n = self.info().n_tasks
        out = np.zeros((n, 8), np.int32)
        self._check(_lib.cp_plan_task_table(self._h, out.ctypes.data, n))
        return out

    def set_epoch(self, epoch: int):
        """Makes the next frame run as ``epoch`` (exercises the epoch wrap)."""
        self._check(_lib.cp_plan_set_epoch(self._h, int(epoch)))

    def set_spin_limit(self, polls: int):
        """Bounds every device-side wait of later frames to ``polls`` reloads
        (0: the default); exercises the time-out path."""
        self._check(_lib.cp_plan_set_spin_limit(self._h, int(polls)))

    def set_crossover(self, rows: int):
        """Frames with fewer than ``rows`` rows run the per-phase executor
        (0: every frame persistent)."""
        self._check(_lib.cp_plan_set_crossover(self._h, int(rows)))

    def device_status(self):
        self._check(_lib.cp_plan_device_status(self._h))

    def close(self):
        if getattr(self, "_h", None):
            _lib.cp_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_io(cfg, inputs: dict, rows=None, device="cuda", logits=True, kv=False):
    """Device frame I/O for synth.make_inputs output."""
    import torch
    rows = inputs["rows"] if rows is None else rows
    hid = np.ascontiguousarray(inputs["hidden"][:rows])
    if hid.dtype == np.uint16:
        hid = hid.view(np.int16)
    io = {
        "rows": rows,
        "hidden_in": torch.from_numpy(hid).to(device),
        "code0": torch.from_numpy(np.ascontiguousarray(inputs["code0"][:rows])).to(device),
        "codes": torch.full((rows, cfg.n_positions - 1), -1, dtype=torch.int32, device=device),
        "embsum": torch.zeros((rows, cfg.hidden), dtype=torch.float32, device=device),
    }
    if logits:
        io["logits"] = torch.zeros((rows, cfg.n_positions - 1, cfg.vocab), dtype=torch.float32, device=device)
    if kv:
        et = torch.int16 if cfg.dtype == "bf16" else torch.float32
        shape = (cfg.n_layers, rows, cfg.n_kv_heads, cfg.n_positions, cfg.head_dim)
        io["k_cache"] = torch.zeros(shape, dtype=et, device=device)
        io["v_cache"] = torch.zeros(shape, dtype=et, device=device)
    if "temperature" in inputs:
        io["temperature"] = torch.from_numpy(np.ascontiguousarray(inputs["temperature"][:rows])).to(device)
        io["top_k"] = torch.from_numpy(np.ascontiguousarray(inputs["top_k"][:rows])).to(device)
        io["top_p"] = torch.from_numpy(np.ascontiguousarray(inputs["top_p"][:rows])).to(device)
        io["seed"] = torch.from_numpy(np.ascontiguousarray(inputs["seed"][:rows]).view(np.int64)).to(device)
        io["offset"] = torch.from_numpy(np.ascontiguousarray(inputs["offset"][:rows]).view(np.int64)).to(device)
    return io
