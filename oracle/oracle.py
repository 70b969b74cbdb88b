"""Python side of the depth-loop CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this module.  It compiles ``oracle.c`` with gcc on first use
and calls it through ctypes; it shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall"]


def build(force: bool = False) -> str:
    """Compiles the oracle library (plain C, gcc) next to its source."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load(path: str):
    """A ctypes handle on an oracle library at `path` (the built one, or a
    copy compiled from altered source by a test that plants a mistake)."""
    l = C.CDLL(path)
    l.orc_frame_run.argtypes = [C.POINTER(_Cfg), C.POINTER(_Weights), C.POINTER(_Frame)]
    l.orc_frame_run.restype = C.c_int
    l.orc_philox4x64.argtypes = [_UP, _UP, _UP]
    l.orc_philox4x64.restype = None
    l.orc_draw.argtypes = [_FP, C.c_int32, C.c_float, C.c_int32, C.c_float, C.c_uint64, C.c_uint64, _DP]
    l.orc_draw.restype = C.c_int32
    l.orc_kept_set.argtypes = [_FP, C.c_int32, C.c_float, C.c_int32, C.c_float, _IP]
    l.orc_kept_set.restype = C.c_int32
    l.orc_round_bf16.argtypes = [C.c_float]
    l.orc_round_bf16.restype = C.c_float
    l.orc_stage_width.argtypes = [C.POINTER(_Cfg)]
    l.orc_stage_width.restype = C.c_int32
    return l


class _Cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "hidden", "input_dim", "n_q_heads",
                                          "n_kv_heads", "head_dim", "intermediate",
                                          "n_positions", "vocab", "bf16")] + [
        ("rms_eps", C.c_double), ("rope_theta", C.c_double), ("qk_norm", C.c_int32)]


_FP = C.POINTER(C.c_float)
_IP = C.POINTER(C.c_int32)
_UP = C.POINTER(C.c_uint64)
_DP = C.POINTER(C.c_double)


class _Weights(C.Structure):
    _fields_ = [(n, _FP) for n in ("w_in", "embed", "attn_norm", "w_qkv", "w_o", "mlp_norm",
                                   "w_gate", "w_up", "w_down", "final_norm", "w_head", "q_norm", "k_norm")]


class _Frame(C.Structure):
    _fields_ = [("rows", C.c_int32), ("hidden_in", _FP), ("code0", _IP),
                ("temperature", _FP), ("top_k", _IP), ("top_p", _FP), ("seed", _UP),
                ("offset_in", _UP), ("forced_codes", _IP), ("codes", _IP), ("embsum", _FP),
                ("logits", _FP), ("k_cache", _FP), ("v_cache", _FP), ("pos_hidden", _FP),
                ("offset_out", _UP), ("margins", _DP), ("n_threads", C.c_int32), ("stages", _FP),
                ("final_normed", _FP)]

# Stages recorded per (row, position, layer) with keep_stages (oracle.h, ORC_ST_*).
STAGES = ("h_in", "a", "qkv_raw", "qkv", "att", "h_mid", "a2", "gate", "up", "m", "h_out")


def lib():
    global _lib
    with _lock:
        if _lib is None:
            _lib = load(build())
    return _lib


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _widen(a, bf16):
    if bf16:
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return _f32(a)


class OracleWeights:
    """Weights widened to float32 and stacked the way ``orc_weights`` wants them.

    ``w`` maps names (``w_in``, ``embed.j``, ``w_qkv.l`` ...) to arrays in the
    storage type; bf16 arrays are uint16 bit patterns.
    """

    def __init__(self, cfg, w: dict):
        bf = cfg.dtype == "bf16"
        L, P = cfg.n_layers, cfg.n_positions
        self.bf16 = bf
        self.arrays = {
            "w_in": _widen(w["w_in"], bf),
            "embed": np.stack([_widen(w[f"embed.{j}"], bf) for j in range(P)]),
            "attn_norm": np.stack([_widen(w[f"attn_norm.{l}"], bf) for l in range(L)]),
            "w_qkv": np.stack([_widen(w[f"w_qkv.{l}"], bf) for l in range(L)]),
            "w_o": np.stack([_widen(w[f"w_o.{l}"], bf) for l in range(L)]),
            "mlp_norm": np.stack([_widen(w[f"mlp_norm.{l}"], bf) for l in range(L)]),
            "w_gate": np.stack([_widen(w[f"w_gate.{l}"], bf) for l in range(L)]),
            "w_up": np.stack([_widen(w[f"w_up.{l}"], bf) for l in range(L)]),
            "w_down": np.stack([_widen(w[f"w_down.{l}"], bf) for l in range(L)]),
            "final_norm": _widen(w["final_norm"], bf),
            "w_head": np.stack([_widen(w[f"w_head.{j}"], bf) for j in range(1, P)]),
        }
        if getattr(cfg, "qk_norm", False):
            self.arrays["q_norm"] = np.stack([_widen(w[f"q_norm.{l}"], bf) for l in range(L)])
            self.arrays["k_norm"] = np.stack([_widen(w[f"k_norm.{l}"], bf) for l in range(L)])
        self.arrays = {k: np.ascontiguousarray(v, np.float32) for k, v in self.arrays.items()}
        self.c = _Weights(**{k: _ptr(v, _FP) for k, v in self.arrays.items()})


def _cfg(cfg):
    return _Cfg(n_layers=cfg.n_layers, hidden=cfg.hidden, input_dim=cfg.input_dim,
                n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                intermediate=cfg.intermediate, n_positions=cfg.n_positions, vocab=cfg.vocab,
                bf16=1 if cfg.dtype == "bf16" else 0, rms_eps=cfg.rms_eps,
                rope_theta=cfg.rope_theta, qk_norm=1 if getattr(cfg, "qk_norm", False) else 0)


def run_frame(cfg, weights, inputs: dict, forced_codes=None, keep_kv: bool = False,
              keep_hidden: bool = False, n_threads: int = 0, rows=None, keep_stages: bool = False,
              library=None) -> dict:
    """One oracle frame.

    ``weights``: an ``OracleWeights`` or a dict of stored weights.  ``inputs``:
    as made by ``synth.make_inputs`` (hidden in the storage type, code0 and,
    when sampling, temperature/top_k/top_p/seed/offset).  ``rows`` optionally
    selects a subset of the input rows (rows are independent).  Returns
    codes [R][P-1], embsum [R][H], logits [R][P-1][V], margins [R][P-1][4],
    offset [R] and, on request, k/v caches [L][R][P][nkv][d], the residual
    stream after the last layer [R][P][H], and (keep_stages) every stage's
    stored values [R][P][L][len(STAGES)][width] with the final-norm outputs
    [R][P-1][H].  ``library``: another oracle library handle (``load``).
    """
    if not isinstance(weights, OracleWeights):
        weights = OracleWeights(cfg, weights)
    bf = cfg.dtype == "bf16"
    sel = np.arange(inputs["rows"]) if rows is None else np.asarray(rows)
    R, P, H, V = len(sel), cfg.n_positions, cfg.hidden, cfg.vocab
    hid = _widen(np.asarray(inputs["hidden"])[sel], bf).reshape(R, cfg.input_dim)
    code0 = np.ascontiguousarray(np.asarray(inputs["code0"])[sel], np.int32)
    out = {
        "codes": np.zeros((R, P - 1), np.int32),
        "embsum": np.zeros((R, H), np.float32),
        "logits": np.zeros((R, P - 1, V), np.float32),
        "margins": np.zeros((R, P - 1, 4), np.float64),
        "offset": np.zeros(R, np.uint64),
    }
    kv_shape = (cfg.n_layers, R, P, cfg.n_kv_heads, cfg.head_dim)
    if keep_kv:
        out["k_cache"] = np.zeros(kv_shape, np.float32)
        out["v_cache"] = np.zeros(kv_shape, np.float32)
    if keep_hidden:
        out["pos_hidden"] = np.zeros((R, P, H), np.float32)
    lb = lib() if library is None else library
    if keep_stages:
        wd = lb.orc_stage_width(C.byref(_cfg(cfg)))
        out["stages"] = np.zeros((R, P, cfg.n_layers, len(STAGES), wd), np.float32)
        out["final_normed"] = np.zeros((R, P - 1, H), np.float32)
    samp = {}
    if "temperature" in inputs:
        samp = {k: np.ascontiguousarray(np.asarray(inputs[k])[sel]) for k in
                ("temperature", "top_k", "top_p", "seed", "offset")}
        samp["temperature"] = samp["temperature"].astype(np.float32)
        samp["top_k"] = samp["top_k"].astype(np.int32)
        samp["top_p"] = samp["top_p"].astype(np.float32)
        samp["seed"] = samp["seed"].astype(np.uint64)
        samp["offset"] = samp["offset"].astype(np.uint64)
    fc = None if forced_codes is None else np.ascontiguousarray(forced_codes, np.int32).reshape(R, P - 1)
    fr = _Frame(rows=R, hidden_in=_ptr(hid, _FP), code0=_ptr(code0, _IP),
                temperature=_ptr(samp.get("temperature"), _FP), top_k=_ptr(samp.get("top_k"), _IP),
                top_p=_ptr(samp.get("top_p"), _FP), seed=_ptr(samp.get("seed"), _UP),
                offset_in=_ptr(samp.get("offset"), _UP), forced_codes=_ptr(fc, _IP),
                codes=_ptr(out["codes"], _IP), embsum=_ptr(out["embsum"], _FP),
                logits=_ptr(out["logits"], _FP), k_cache=_ptr(out.get("k_cache"), _FP),
                v_cache=_ptr(out.get("v_cache"), _FP), pos_hidden=_ptr(out.get("pos_hidden"), _FP),
                offset_out=_ptr(out["offset"], _UP), margins=_ptr(out["margins"], _DP),
                n_threads=int(n_threads), stages=_ptr(out.get("stages"), _FP),
                final_normed=_ptr(out.get("final_normed"), _FP))
        # keep numpy buffers alive for the duration of the call
    keep = (hid, code0, samp, fc, weights)
    rc = lb.orc_frame_run(C.byref(_cfg(cfg)), C.byref(weights.c), C.byref(fr))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the frame (code {rc})")
    return out


def philox4x64(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, np.uint64)
    k = np.ascontiguousarray(key, np.uint64)
    o = np.zeros(4, np.uint64)
    lib().orc_philox4x64(_ptr(c, _UP), _ptr(k, _UP), _ptr(o, _UP))
    return o


def draw(z, temperature=0.0, top_k=0, top_p=1.0, seed=0, counter=0):
    """One draw from logits z; returns (code, margins[4])."""
    zz = _f32(z)
    m = np.zeros(4, np.float64)
    code = lib().orc_draw(_ptr(zz, _FP), len(zz), float(temperature), int(top_k), float(top_p),
                          int(seed), int(counter), _ptr(m, _DP))
    return int(code), m


def kept_set(z, temperature, top_k, top_p) -> np.ndarray:
    zz = _f32(z)
    kept = np.zeros(len(zz), np.int32)
    n = lib().orc_kept_set(_ptr(zz, _FP), len(zz), float(temperature), int(top_k), float(top_p),
                           _ptr(kept, _IP))
    return kept[:n].copy()


def round_bf16(x: float) -> float:
    return float(lib().orc_round_bf16(float(x)))
