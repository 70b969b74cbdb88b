"""Seeded synthetic workloads for the codec-TTS depth loop.

This module only draws random numbers and stores them in the storage type of a
configuration (fp32, or bf16 held as uint16 bit patterns).  It holds none of
the depth loop's arithmetic: the CPU oracle and the HIP library both take what
it produces as plain inputs.

Shapes follow the depth loop of the "Qwen3-TTS: run the 1.7B depth loop as one
persistent kernel on Hopper" pull request (mstar #1183), section "How it works":
an N-layer decoder over 16 depth positions with 15 code heads; hidden 1024,
16 query and 8 key/value heads of 128, SwiGLU intermediate 3072.  Real weights
and real Talker hidden states are not available, so every tensor is drawn from
a fixed seeded distribution instead:

* weight matrices and embedding tables ~ N(0, 0.02);
* RMSNorm gains 1.0 (or 1 + N(0, 0.1) in the test-only ``gain_jitter`` variant),
  the per-head q and k norm gains of the QK-norm variant included;
* the input hidden ~ N(0, 1), one independent vector per row;
* code 0 (supplied by the Talker in the real model) ~ U[0, vocab);
* sampling parameters per row: temperature ~ U[0.6, 1.2], top-k uniform in
  {10, 20, 50}, top-p ~ U[0.8, 0.95], a 64-bit Philox seed and a 32-bit offset.

Every tensor comes from its own generator, ``PCG64(SeedSequence([seed, tag,
idx]))``, so any row or tensor can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

TAG_WEIGHT = 0
TAG_HIDDEN = 1
TAG_CODE0 = 2
TAG_SAMPLING = 3
TAG_GAIN = 4


@dataclass(frozen=True)
class DepthLoopConfig:
    """Shapes of one depth-loop workload (one frame over ``rows`` requests)."""

    name: str
    n_layers: int
    hidden: int
    input_dim: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    n_positions: int
    vocab: int
    dtype: str  # "f32" or "bf16": storage and activation type
    rows: int
    sampled: bool = False
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    qk_norm: bool = False  # Qwen3-style RMSNorm of each q and k head before RoPE

    @property
    def n_heads_out(self) -> int:
        """Code heads: one per position after the first."""
        return self.n_positions - 1

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_(self, **kw) -> "DepthLoopConfig":
        return dataclasses.replace(self, **kw)

    def layer_weight_bytes(self) -> int:
        """Bytes of one layer's projection weights in the storage type."""
        esz = 4 if self.dtype == "f32" else 2
        h, i = self.hidden, self.intermediate
        qd = self.n_q_heads * self.head_dim
        return esz * (self.qkv_dim * h + h * qd + 2 * i * h + h * i)

    def frame_weight_bytes(self) -> int:
        """Algorithmic weight bytes of one frame.

        Every position re-reads all layer weights; the input projection and
        each code head are read once.  Norm gains, embedding rows and the KV
        cache are left out (each is under 1% of the total).
        """
        esz = 4 if self.dtype == "f32" else 2
        return (self.n_positions * self.n_layers * self.layer_weight_bytes()
                + esz * self.hidden * self.input_dim
                + esz * self.n_heads_out * self.vocab * self.hidden)

    def frame_flops(self) -> int:
        """Multiply-add FLOPs of the projections for all rows of one frame."""
        esz = 4 if self.dtype == "f32" else 2
        return 2 * self.rows * (self.frame_weight_bytes() // esz)


_FULL = dict(n_layers=5, hidden=1024, input_dim=1024, n_q_heads=16, n_kv_heads=8,
             head_dim=128, intermediate=3072, n_positions=16, vocab=2048, dtype="bf16")

CONFIGS: dict[str, DepthLoopConfig] = {
    # Tiny fp32 depth loop used for tight correctness checks.
    "tiny_f32": DepthLoopConfig(name="tiny_f32", n_layers=2, hidden=256, input_dim=256,
                                n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=768,
                                n_positions=4, vocab=256, dtype="f32", rows=1),
    # Full-size 5-layer bf16 depth loop (157 MB of layer weights).
    "l5_r1": DepthLoopConfig(name="l5_r1", rows=1, **_FULL),
    "l5_r64": DepthLoopConfig(name="l5_r64", rows=64, **_FULL),
    "l5_r64_sampled": DepthLoopConfig(name="l5_r64_sampled", rows=64, sampled=True, **_FULL),
    # A frame of 128 rows (two groups of 64 per projection task).
    "l5_r128": DepthLoopConfig(name="l5_r128", rows=128, **_FULL),
    # 10-layer variant: 314 MB of layer weights, more than the 256 MB Infinity Cache.
    "l10_r1": DepthLoopConfig(name="l10_r1", rows=1, **{**_FULL, "n_layers": 10}),
    "l10_r16": DepthLoopConfig(name="l10_r16", rows=16, **{**_FULL, "n_layers": 10}),
    "l10_r64": DepthLoopConfig(name="l10_r64", rows=64, **{**_FULL, "n_layers": 10}),
    # Qwen3-style variant: RMSNorm of every q and k head before RoPE.
    "l5_qk_r64": DepthLoopConfig(name="l5_qk_r64", rows=64, qk_norm=True, **_FULL),
    # Input projection from a 2048-wide hidden (a larger text model) to 1024.
    "l5_in2048_r8": DepthLoopConfig(name="l5_in2048_r8", rows=8, **{**_FULL, "input_dim": 2048}),
}


def _rng(seed: int, tag: int, idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, idx])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even), as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.isfinite(x).all():
        raise ValueError("non-finite value in a synthetic tensor")
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(cfg: DepthLoopConfig, a: np.ndarray) -> np.ndarray:
    """A stored tensor as float32 values (widening bf16 bit patterns exactly)."""
    return bf16_bits_to_f32(a) if cfg.dtype == "bf16" else np.asarray(a, dtype=np.float32)


def _store(cfg: DepthLoopConfig, x: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x) if cfg.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _normal(cfg, seed, tag, idx, shape, std):
    x = _rng(seed, tag, idx).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _store(cfg, x)


def weight_names(cfg: DepthLoopConfig) -> list[str]:
    """Matrices in their canonical seeding order (the ``idx`` of each generator)."""
    names = ["w_in"] + [f"embed.{j}" for j in range(cfg.n_positions)]
    for l in range(cfg.n_layers):
        names += [f"w_qkv.{l}", f"w_o.{l}", f"w_gate.{l}", f"w_up.{l}", f"w_down.{l}"]
    names += [f"w_head.{j}" for j in range(1, cfg.n_positions)]
    return names


def weight_shape(cfg: DepthLoopConfig, name: str) -> tuple[int, int]:
    """Row-major [out][in] shape, as nn.Linear stores it; embeddings are [vocab][hidden]."""
    kind = name.split(".")[0]
    h, i, qd = cfg.hidden, cfg.intermediate, cfg.n_q_heads * cfg.head_dim
    return {
        "w_in": (h, cfg.input_dim),
        "embed": (cfg.vocab, h),
        "w_qkv": (cfg.qkv_dim, h),  # rows: q heads, then k heads, then v heads
        "w_o": (h, qd),
        "w_gate": (i, h),
        "w_up": (i, h),
        "w_down": (h, i),
        "w_head": (cfg.vocab, h),
    }[kind]


def make_weights(cfg: DepthLoopConfig, seed: int = 0, gain_jitter: bool = False) -> dict:
    """All weights of one configuration, keyed by name, in the storage type.

    Matrices are ``weight_names`` order; norm gains are ``attn_norm.l``,
    ``mlp_norm.l`` and ``final_norm`` of length ``hidden`` and, with
    ``qk_norm``, ``q_norm.l`` and ``k_norm.l`` of length ``head_dim``.
    """
    w = {}
    for idx, name in enumerate(weight_names(cfg)):
        w[name] = _normal(cfg, seed, TAG_WEIGHT, idx, weight_shape(cfg, name), 0.02)
    for l in range(cfg.n_layers):
        for k, nm in enumerate(("attn_norm", "mlp_norm")):
            g = np.ones(cfg.hidden, np.float32)
            if gain_jitter:
                g += _rng(seed, TAG_GAIN, 2 * l + k).standard_normal(cfg.hidden, dtype=np.float32) * np.float32(0.1)
            w[f"{nm}.{l}"] = _store(cfg, g)
    g = np.ones(cfg.hidden, np.float32)
    if gain_jitter:
        g += _rng(seed, TAG_GAIN, 2 * cfg.n_layers).standard_normal(cfg.hidden, dtype=np.float32) * np.float32(0.1)
    w["final_norm"] = _store(cfg, g)
    if cfg.qk_norm:
        for l in range(cfg.n_layers):
            for k, nm in enumerate(("q_norm", "k_norm")):
                g = np.ones(cfg.head_dim, np.float32)
                if gain_jitter:
                    g += _rng(seed, TAG_GAIN, 2 * cfg.n_layers + 1 + 2 * l + k).standard_normal(
                        cfg.head_dim, dtype=np.float32) * np.float32(0.1)
                w[f"{nm}.{l}"] = _store(cfg, g)
    return w


def make_inputs(cfg: DepthLoopConfig, rows: int | None = None, seed: int = 0,
                sampled: bool | None = None) -> dict:
    """Per-row frame inputs: hidden [rows][input_dim], code0 [rows] and, when
    sampling, temperature / top_k / top_p / seed / offset [rows]."""
    rows = cfg.rows if rows is None else rows
    sampled = cfg.sampled if sampled is None else sampled
    hid = np.stack([_rng(seed, TAG_HIDDEN, r).standard_normal(cfg.input_dim, dtype=np.float32)
                    for r in range(rows)]) if rows else np.zeros((0, cfg.input_dim), np.float32)
    out = {
        "rows": rows,
        "hidden": _store(cfg, hid),
        "code0": np.array([_rng(seed, TAG_CODE0, r).integers(0, cfg.vocab) for r in range(rows)],
                          dtype=np.int32),
    }
    if sampled:
        t, k, p, s, o = [], [], [], [], []
        for r in range(rows):
            g = _rng(seed, TAG_SAMPLING, r)
            t.append(g.uniform(0.6, 1.2))
            k.append(g.choice([10, 20, 50]))
            p.append(g.uniform(0.8, 0.95))
            s.append(g.integers(0, 2**64, dtype=np.uint64))
            o.append(g.integers(0, 2**32, dtype=np.uint64))
        out.update(temperature=np.array(t, np.float32), top_k=np.array(k, np.int32),
                   top_p=np.array(p, np.float32), seed=np.array(s, np.uint64),
                   offset=np.array(o, np.uint64))
    return out
