"""Pins of where the CPU oracle rounds to bf16 (and where it must not).

The depth loop's frame (mstar pull request #1183, "Qwen3-TTS: Run the 1.7B
Depth Loop as One Persistent Kernel on Hopper", section "How it works") keeps
its activations in bf16: the normed activation before each projection, q / k /
v after RoPE, the attention output, the residual after o and after down, the
SwiGLU output and the final-norm output are stored rounded; projection
outputs feeding a nonlinearity (gate, up), softmax weights and the logits
stay fp32 (section "Testing" compares the logits as floats).

Three kinds of checks:
  * every stage the oracle records is recomputed here from the stage before
    it, in float64 with numpy (products of two floats are exact in float64;
    sums in the oracle's order), rounded to float32 by numpy and to bf16 by
    torch, and must equal the oracle's value bit for bit;
  * a planted one-layer frame whose rounded values are worked out by hand;
  * mutants of oracle.c, each with one rounding removed, moved or added,
    compiled here: every one must fail the checks above.
"""
import math
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from persistent_megakernel_streaming_amd import synth

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")


# ------------------------------------------------------------------ reference arithmetic

def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


def _bf(x32):
    """float32 -> bf16 (round to nearest even, by torch) -> float32."""
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _dot(W, x):
    """W . x in float64, each row summed left to right (the oracle's order)."""
    prod = np.asarray(W, np.float64) * np.asarray(x, np.float64)[None, :]
    return np.add.accumulate(prod, axis=1)[:, -1]


def _store(cfg, x64):
    return _bf(_f32(x64)) if cfg.dtype == "bf16" else _f32(x64)


def _undecided(cfg, x64):
    """Elements within 1e-13 (relative) of a rounding boundary: the last
    double-rounding step cannot be decided from a differently ordered
    transcendental (none expected; counted)."""
    x64 = np.asarray(x64, np.float64)
    return _store(cfg, x64 * (1 - 1e-13)) != _store(cfg, x64 * (1 + 1e-13))


def _rmsnorm(cfg, h, g):
    ss = 0.0
    for v in np.asarray(h, np.float64):
        ss += v * v
    r = np.float32(1.0 / math.sqrt(ss / len(h) + cfg.rms_eps))
    t = np.asarray(h, np.float32) * r
    v = t * np.asarray(g, np.float32)
    return _bf(v) if cfg.dtype == "bf16" else v


def stage_failures(cfg, w, inp, out):
    """Recomputes each recorded stage from the one before it; returns a list
    of (stage, row, position, layer, mismatches) and the undecided count."""
    ow = {k: (synth.as_f32(cfg, v)) for k, v in w.items()}
    L, P, H = cfg.n_layers, cfg.n_positions, cfg.hidden
    nq, nkv, d, I = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    qd, half = nq * d, d // 2
    st = out["stages"]
    S = {n: i for i, n in enumerate(("h_in", "a", "qkv_raw", "qkv", "att", "h_mid", "a2", "gate", "up", "m", "h_out"))}
    bad, und = [], 0

    def cmp(name, r, p, l, got, exp64=None, exp=None):
        nonlocal und
        if exp is None:
            exp = _store(cfg, exp64)
            u = _undecided(cfg, exp64)
            und += int(u.sum())
        else:
            u = np.zeros(len(exp), bool)
        n = int(np.sum((got.view(np.uint32) != np.asarray(exp, np.float32).view(np.uint32)) & ~u))
        if n:
            bad.append((name, r, p, l, n))

    cs = np.zeros((P, half), np.float32)
    sn = np.zeros((P, half), np.float32)
    for p in range(P):
        for i in range(half):
            ang = p * math.pow(cfg.rope_theta, -2.0 * i / d)
            cs[p, i], sn[p, i] = np.float32(math.cos(ang)), np.float32(math.sin(ang))
    x = synth.as_f32(cfg, inp["hidden"])
    for r in range(inp["rows"]):
        for p in range(P):
            for l in range(L):
                g = lambda n, k=None: st[r, p, l, S[n], :k]
                h_in = g("h_in", H)
                if l == 0:
                    if p == 0:
                        cmp("input projection", r, p, l, h_in, exp64=_dot(ow["w_in"], x[r]))
                    else:
                        code = inp["code0"][r] if p == 1 else out["codes"][r, p - 2]
                        cmp("position input", r, p, l, h_in, exp=ow[f"embed.{p - 1}"][code])
                else:
                    cmp("layer input", r, p, l, h_in, exp=st[r, p, l - 1, S["h_out"], :H])
                a = g("a", H)
                cmp("attention norm", r, p, l, a, exp=_rmsnorm(cfg, h_in, ow[f"attn_norm.{l}"]))
                raw = g("qkv_raw", (nq + 2 * nkv) * d)
                cmp("qkv projection", r, p, l, raw, exp=_f32(_dot(ow[f"w_qkv.{l}"], a)))
                rot = np.asarray(raw, np.float64).copy()
                for hd in range(nq + nkv):
                    x1 = raw[hd * d:hd * d + half].astype(np.float64)
                    x2 = raw[hd * d + half:(hd + 1) * d].astype(np.float64)
                    c, s = cs[p].astype(np.float64), sn[p].astype(np.float64)
                    rot[hd * d:hd * d + half] = _f32(x1 * c - x2 * s)
                    rot[hd * d + half:(hd + 1) * d] = _f32(x2 * c + x1 * s)
                cmp("q, k, v after RoPE", r, p, l, g("qkv", (nq + 2 * nkv) * d), exp64=rot)
                qkv = [st[r, t, l, S["qkv"], :(nq + 2 * nkv) * d] for t in range(p + 1)]
                att = np.zeros(qd)
                for hq in range(nq):
                    kv = hq // (nq // nkv)
                    q = qkv[p][hq * d:(hq + 1) * d]
                    sc = [_dot(qkv[t][qd + kv * d:qd + (kv + 1) * d][None, :], q)[0] / math.sqrt(d)
                          for t in range(p + 1)]
                    mx = max(sc)
                    e = [math.exp(s - mx) for s in sc]
                    zs = 0.0
                    for v in e:
                        zs += v
                    for i in range(d):
                        o = 0.0
                        for t in range(p + 1):
                            o += (e[t] / zs) * float(qkv[t][qd + (nkv + kv) * d + i])
                        att[hq * d + i] = o
                a_st = g("att", qd)
                cmp("attention output", r, p, l, a_st, exp64=att)
                hm = g("h_mid", H)
                cmp("residual after o", r, p, l, hm, exp64=h_in.astype(np.float64) + _dot(ow[f"w_o.{l}"], a_st))
                a2 = g("a2", H)
                cmp("MLP norm", r, p, l, a2, exp=_rmsnorm(cfg, hm, ow[f"mlp_norm.{l}"]))
                gt, up = g("gate", I), g("up", I)
                cmp("gate", r, p, l, gt, exp=_f32(_dot(ow[f"w_gate.{l}"], a2)))
                cmp("up", r, p, l, up, exp=_f32(_dot(ow[f"w_up.{l}"], a2)))
                gv = gt.astype(np.float64)
                sl = np.array([v / (1.0 + math.exp(-v)) for v in gv])
                m = g("m", I)
                cmp("SwiGLU output", r, p, l, m, exp64=sl * up.astype(np.float64))
                cmp("residual after down", r, p, l, g("h_out", H),
                    exp64=hm.astype(np.float64) + _dot(ow[f"w_down.{l}"], m))
            if p >= 1:
                f = out["final_normed"][r, p - 1]
                cmp("final norm", r, p, -1, f, exp=_rmsnorm(cfg, st[r, p, L - 1, S["h_out"], :H], ow["final_norm"]))
                cmp("logits (float, not rounded)", r, p, -1, out["logits"][r, p - 1],
                    exp=_f32(_dot(ow[f"w_head.{p}"], f)))
    return bad, und


# ------------------------------------------------------------------ planted frame

def planted():
    """One layer, hidden 4, one q and one kv head of 4, SwiGLU width 4, three
    positions, vocab 4, bf16, epsilon 0.  Position 0's input is x = [2, 1, 1,
    1] through W_in = I; position 1's is E_0[c_0] = [1, 1, 1, 2]; position 2's
    is any row of E_1 = [3, 3, 1, 1] (all rows alike, so the drawn code does
    not matter).  W_q = 0 (every score 0: uniform attention), W_k = I, W_v row
    0 = [1, -1, 0, 0] and the other v rows 0, W_o = I, W_gate = 0, W_up = I,
    W_down = I; gains 1."""
    cfg = synth.CONFIGS["tiny_f32"].with_(n_layers=1, hidden=4, input_dim=4, n_q_heads=1, n_kv_heads=1,
                                          head_dim=4, intermediate=4, n_positions=3, vocab=4, dtype="bf16",
                                          rows=1, rms_eps=0.0)
    bf = lambda a: synth.f32_to_bf16_bits(np.asarray(a, np.float32))
    eye, z4 = np.eye(4, dtype=np.float32), np.zeros((4, 4), np.float32)
    wv = np.zeros((4, 4), np.float32)
    wv[0] = [1, -1, 0, 0]
    w = {"w_in": bf(eye), "final_norm": bf(np.ones(4)),
         "embed.0": bf(np.tile([1, 1, 1, 2], (4, 1))), "embed.1": bf(np.tile([3, 3, 1, 1], (4, 1))),
         "embed.2": bf(np.tile([1, 2, 3, 4], (4, 1))),
         "attn_norm.0": bf(np.ones(4)), "mlp_norm.0": bf(np.ones(4)),
         "w_qkv.0": bf(np.concatenate([z4, eye, wv])), "w_o.0": bf(eye), "w_gate.0": bf(z4),
         "w_up.0": bf(eye), "w_down.0": bf(eye),
         "w_head.1": bf(eye), "w_head.2": bf(eye)}
    inp = {"rows": 1, "hidden": bf(np.array([[2, 1, 1, 1]])), "code0": np.array([0], np.int32)}
    return cfg, w, inp


def planted_failures(out):
    """Values of the planted frame worked out by hand (bf16 keeps 8
    significant bits; ties go to the even neighbour):
      * position 1's attention norm: mean(h^2) = 7/4, so h / rms =
        [2/sqrt 7] * 3 + [4/sqrt 7] = [0.755929, ..] and [1.511858]; in bf16
        0.755929 = 1.511858 / 2 and 1.511858 * 128 = 193.52 -> 194, so
        a = [0.7578125] * 3 + [1.515625];
      * position 0 (h = [2, 1, 1, 1]): a = [1.515625, 0.7578125, 0.7578125,
        0.7578125], so V_0[0] = bf(a0 - a1) = 0.7578125, and position 0's
        attention output is V_0 itself (one key, weight 1);
      * V_1[0] = V_2[0] = 0 (a0 = a1 there); at position 2 the three scores
        are equal, so att[0] = bf(0.7578125 / 3) = bf(0.2526042): 0.2526042 * 4
        = 1.0104167, * 128 = 129.33 -> 129, att[0] = 129 / 512 = 0.251953125;
      * the residual after o at position 2, channel 0: 3 + 0.251953125 =
        3.251953125; bf16 has 2^-6 steps in [2, 4): 3.251953125 * 64 = 208.125
        -> 208, so 3.25;
      * W_gate = 0: silu(0) = 0, so the SwiGLU output is exactly 0 and the
        residual after down equals the residual after o."""
    st = out["stages"][0]
    bad = []
    checks = [
        ("attention norm, position 1", st[1, 0, 1, :4], [0.7578125, 0.7578125, 0.7578125, 1.515625]),
        ("attention norm, position 0", st[0, 0, 1, :4], [1.515625, 0.7578125, 0.7578125, 0.7578125]),
        ("v_0 channel 0", st[0, 0, 3, 8:9], [0.7578125]),
        ("attention output, position 0 = V_0", st[0, 0, 4, :4], st[0, 0, 3, 8:12]),
        ("attention output, position 2", st[2, 0, 4, :1], [0.251953125]),
        ("residual after o, position 2", st[2, 0, 5, :1], [3.25]),
        ("SwiGLU output", st[:, 0, 9, :4], np.zeros((3, 4))),
        ("residual after down", st[:, 0, 10, :4], st[:, 0, 5, :4]),
    ]
    for name, got, exp in checks:
        if not np.array_equal(np.asarray(got, np.float32), np.asarray(exp, np.float32)):
            bad.append((name, np.asarray(got).tolist()))
    return bad


def _random_frame():
    cfg = synth.CONFIGS["tiny_f32"].with_(rows=2, dtype="bf16", n_positions=4)
    w = synth.make_weights(cfg, seed=31, gain_jitter=True)
    inp = synth.make_inputs(cfg, seed=31)
    return cfg, w, inp


def _run_checks(oracle_mod, library=None):
    problems = []
    for cfg, w, inp in (_random_frame(), planted()):
        out = oracle_mod.run_frame(cfg, w, inp, keep_stages=True, library=library)
        bad, und = stage_failures(cfg, w, inp, out)
        problems += bad
        assert und <= 2, und
    cfg, w, inp = planted()
    problems += planted_failures(oracle_mod.run_frame(cfg, w, inp, keep_stages=True, library=library))
    return problems


# ------------------------------------------------------------------ tests

def test_oracle_rounds_exactly_where_defined(oracle_mod):
    assert _run_checks(oracle_mod) == []


def test_oracle_fp32_stages_are_unrounded(oracle_mod):
    """In the fp32 configuration the same stages hold plain float values."""
    cfg = synth.CONFIGS["tiny_f32"].with_(rows=2, n_positions=3)
    w = synth.make_weights(cfg, seed=32, gain_jitter=True)
    inp = synth.make_inputs(cfg, seed=32)
    out = oracle_mod.run_frame(cfg, w, inp, keep_stages=True)
    bad, und = stage_failures(cfg, w, inp, out)
    assert bad == [] and und <= 2


# Each mutant: (name, [(pattern, replacement)]) applied to oracle.c; every
# pattern must occur exactly once.
MUTANTS = [
    ("norm: no rounding", [(r"out\[i\] = c->bf16 \? orc_round_bf16\(v\) : v;", "out[i] = v;")]),
    ("norm: rounds h*r before the gain",
     [(r"float t = h\[i\] \* r;", "float t = c->bf16 ? orc_round_bf16(h[i] * r) : h[i] * r;"),
      (r"out\[i\] = c->bf16 \? orc_round_bf16\(v\) : v;", "out[i] = v;")]),
    ("input projection: no rounding", [(r"store_act\(c, dot\(w->w_in", "(float)(dot(w->w_in")]),
    ("qkv: no rounding", [(r"row\[n\] = store_act\(c, row\[n\]\);", "row[n] = row[n];")]),
    ("qkv: rounds before RoPE",
     [(r"qkv\[\(size_t\)r \* QKV \+ n\] = \(float\)dot\(", "qkv[(size_t)r * QKV + n] = store_act(c, dot("),
      (r"a \+ \(size_t\)r \* H, H\);\n      record\(c, fr, p, l, ORC_ST_QKV_RAW",
       "a + (size_t)r * H, H));\n      record(c, fr, p, l, ORC_ST_QKV_RAW"),
      (r"row\[n\] = store_act\(c, row\[n\]\);", "row[n] = row[n];")]),
    ("attention: no rounding", [(r"= store_act\(c, o\);", "= (float)(o);")]),
    ("attention: rounds the softmax weights instead",
     [(r"o \+= \(ep\[t\] / zs\)", "o += (double)orc_round_bf16((float)(ep[t] / zs))"),
      (r"= store_act\(c, o\);", "= (float)(o);")]),
    ("residual after o: no rounding",
     [(r"store_act\(c, v\); /\* a used as scratch for the new h \*/", "(float)(v);")]),
    ("residual after o: rounds the product before the add",
     [(r"double v = \(double\)h\[\(size_t\)r \* H \+ n\] \+ dot\(wo \+ \(size_t\)n \* qd, att \+ \(size_t\)r \* qd, qd\);",
       "double v = (double)h[(size_t)r * H + n] + (double)store_act(c, dot(wo + (size_t)n * qd, att + (size_t)r * qd, qd));"),
      (r"store_act\(c, v\); /\* a used as scratch for the new h \*/", "(float)(v);")]),
    ("SwiGLU: no rounding", [(r"store_act\(c, sl \* \(double\)uv\)", "(float)(sl * (double)uv)")]),
    ("SwiGLU: rounds gate and up instead",
     [(r"float gv = \(float\)dot\(", "float gv = store_act(c, dot("),
      (r"float uv = \(float\)dot\(", "float uv = store_act(c, dot("),
      (r"\(size_t\)n \* H, a \+ \(size_t\)r \* H, H\);\n          float uv",
       "(size_t)n * H, a + (size_t)r * H, H));\n          float uv"),
      (r"\(size_t\)n \* H, a \+ \(size_t\)r \* H, H\);\n          double sl",
       "(size_t)n * H, a + (size_t)r * H, H));\n          double sl"),
      (r"store_act\(c, sl \* \(double\)uv\)", "(float)(sl * (double)uv)")]),
    ("residual after down: no rounding",
     [(r"a\[\(size_t\)r \* H \+ n\] = store_act\(c, v\);\n        \}\n      memcpy\(h, a, sizeof\(float\) \* \(size_t\)R \* H\);\n      record\(c, fr, p, l, ORC_ST_H_OUT",
       "a[(size_t)r * H + n] = (float)(v);\n        }\n      memcpy(h, a, sizeof(float) * (size_t)R * H);\n      record(c, fr, p, l, ORC_ST_H_OUT")]),
    ("logits: rounded", [(r"z\[\(size_t\)r \* V \+ n\] = \(float\)dot\(wh \+ \(size_t\)n \* H, a \+ \(size_t\)r \* H, H\);",
                          "z[(size_t)r * V + n] = store_act(c, dot(wh + (size_t)n * H, a + (size_t)r * H, H));")]),
]


def _mutant_source(edits):
    src = open(ORACLE_SRC).read()
    for pat, rep in edits:
        n = len(re.findall(pat, src))
        assert n == 1, (pat, n)
        src = re.sub(pat, lambda _m: rep, src)
    return src


def test_every_rounding_mutant_fails_the_pins(oracle_mod, tmp_path):
    """Planting a mistake in the oracle (on the CPU): removing, moving or
    adding any one rounding makes the checks above fail."""
    hdr = os.path.dirname(ORACLE_SRC)
    survivors = []
    for i, (name, edits) in enumerate(MUTANTS):
        c = tmp_path / f"mut{i}.c"
        c.write_text(_mutant_source(edits))
        so = tmp_path / f"libmut{i}.so"
        subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               "-I", hdr, "-o", str(so), str(c), "-lm"])
        lib = oracle_mod.load(str(so))
        try:
            problems = _run_checks(oracle_mod, library=lib)
        except AssertionError:
            problems = ["undecided"]
        if not problems:
            survivors.append(name)
    assert survivors == [], survivors
