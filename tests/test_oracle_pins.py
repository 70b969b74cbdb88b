"""Pins of the CPU oracle against things other than itself.

* The decoder stack (RMSNorm, rotate-half RoPE, grouped-query causal attention,
  SwiGLU, residuals, final norm) against an fp64 Llama forward from the
  ``transformers`` library, fed the frame's 16 inputs with teacher forcing.
* Philox4x64-10 against numpy's independent ``Philox`` bit generator.
* bf16 rounding against torch's float32 -> bfloat16 conversion.
* The draw against the definition of top-k / top-p sets and against the
  Gumbel-max sampling law (chi-square on the empirical code frequencies).
* The frame's wiring (which head reads which position, which table embeds
  which code, causality over positions, the embedding sum, the offsets).

The method is the depth loop of mstar pull request #1183, "Qwen3-TTS: Run the
1.7B Depth Loop as One Persistent Kernel on Hopper", section "How it works"
(phase list; per-row sampler parameters; offsets advance once per draw) and
section "Testing" (codes and embedding sums compared exactly, KV and logits
with tolerances).
"""
import json
import os

import numpy as np
import pytest
import torch

from persistent_megakernel_streaming_amd import synth

TINY = synth.CONFIGS["tiny_f32"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers

def _hf_model(cfg, w):
    """The transformers stack of the same shapes: Llama, or Qwen3 (whose
    attention norms every q and k head before RoPE) for the QK-norm variant."""
    kw = dict(vocab_size=cfg.vocab, hidden_size=cfg.hidden,
              intermediate_size=cfg.intermediate, num_hidden_layers=cfg.n_layers,
              num_attention_heads=cfg.n_q_heads, num_key_value_heads=cfg.n_kv_heads,
              head_dim=cfg.head_dim, rms_norm_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
              max_position_embeddings=64, attention_bias=False,
              tie_word_embeddings=False, attn_implementation="eager")
    if cfg.qk_norm:
        from transformers import Qwen3Config, Qwen3Model
        m = Qwen3Model(Qwen3Config(**kw)).double().eval()
    else:
        from transformers import LlamaConfig, LlamaModel
        m = LlamaModel(LlamaConfig(mlp_bias=False, **kw)).double().eval()
    f = lambda a: torch.from_numpy(synth.as_f32(cfg, a).astype(np.float64))
    sd = m.state_dict()
    qd, kd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    for l in range(cfg.n_layers):
        qkv = f(w[f"w_qkv.{l}"])
        p = f"layers.{l}."
        sd[p + "self_attn.q_proj.weight"] = qkv[:qd]
        sd[p + "self_attn.k_proj.weight"] = qkv[qd:qd + kd]
        sd[p + "self_attn.v_proj.weight"] = qkv[qd + kd:]
        sd[p + "self_attn.o_proj.weight"] = f(w[f"w_o.{l}"])
        sd[p + "mlp.gate_proj.weight"] = f(w[f"w_gate.{l}"])
        sd[p + "mlp.up_proj.weight"] = f(w[f"w_up.{l}"])
        sd[p + "mlp.down_proj.weight"] = f(w[f"w_down.{l}"])
        sd[p + "input_layernorm.weight"] = f(w[f"attn_norm.{l}"])
        sd[p + "post_attention_layernorm.weight"] = f(w[f"mlp_norm.{l}"])
        if cfg.qk_norm:
            sd[p + "self_attn.q_norm.weight"] = f(w[f"q_norm.{l}"])
            sd[p + "self_attn.k_norm.weight"] = f(w[f"k_norm.{l}"])
    sd["norm.weight"] = f(w["final_norm"])
    m.load_state_dict(sd)
    return m, f


def _hf_frame(cfg, w, inp, r, codes):
    """Teacher-forced frame of row r through the transformers Llama stack:
    position 0 = W_in x, position 1 = E_0[code0], position j+1 = E_j[c_j];
    head j reads position j after the final norm."""
    m, f = _hf_model(cfg, w)
    P = cfg.n_positions
    x = f(inp["hidden"][r])
    allc = [int(inp["code0"][r])] + [int(c) for c in codes]
    embs = [f(w["w_in"]) @ x] + [f(w[f"embed.{j}"])[allc[j]] for j in range(P - 1)]
    with torch.no_grad():
        o = m(inputs_embeds=torch.stack(embs)[None], use_cache=True)
    hn = o.last_hidden_state[0]
    z = np.stack([(f(w[f"w_head.{j}"]) @ hn[j]).numpy() for j in range(1, P)])
    kv = o.past_key_values
    ks = np.stack([kv.layers[l].keys[0].numpy() for l in range(cfg.n_layers)])    # [L][nkv][P][d]
    vs = np.stack([kv.layers[l].values[0].numpy() for l in range(cfg.n_layers)])
    return z, ks, vs


# ------------------------------------------------------------------ transformer stack

@pytest.mark.parametrize("variant", [
    dict(),                                           # tiny fp32 shapes
    dict(input_dim=192),                              # input projection is [hidden][input_dim]
    dict(n_kv_heads=4),                               # plain multi-head attention
    dict(n_kv_heads=1, n_positions=6, vocab=64),      # one kv head, more positions
])
def test_oracle_matches_transformers_llama_fp64(oracle_mod, variant):
    cfg = TINY.with_(rows=3, **variant)
    w = synth.make_weights(cfg, seed=11, gain_jitter=True)
    inp = synth.make_inputs(cfg, seed=11)
    out = oracle_mod.run_frame(cfg, w, inp, keep_kv=True)
    for r in range(cfg.rows):
        z, ks, vs = _hf_frame(cfg, w, inp, r, out["codes"][r])
        scale = np.abs(z).max()
        assert np.abs(out["logits"][r] - z).max() <= 2e-6 * max(1.0, scale)
        k_or = out["k_cache"][:, r].transpose(0, 2, 1, 3)  # [L][nkv][P][d]
        v_or = out["v_cache"][:, r].transpose(0, 2, 1, 3)
        assert np.abs(k_or - ks).max() <= 2e-6 * max(1.0, np.abs(ks).max())
        assert np.abs(v_or - vs).max() <= 2e-6 * max(1.0, np.abs(vs).max())


@pytest.mark.parametrize("variant", [
    dict(),                                           # tiny fp32 shapes
    dict(n_kv_heads=1, n_positions=6, vocab=64),      # one kv head, more positions
    dict(head_dim=128, n_q_heads=2, n_kv_heads=2),    # the full model's head size
])
def test_oracle_qk_norm_matches_transformers_qwen3_fp64(oracle_mod, variant):
    """The QK-norm variant (per-head RMSNorm of q and k with their own gains,
    before RoPE) against transformers' Qwen3 stack in fp64, with jittered
    gains so that q_norm and k_norm cannot be swapped or dropped unseen."""
    cfg = TINY.with_(rows=2, qk_norm=True, **variant)
    w = synth.make_weights(cfg, seed=13, gain_jitter=True)
    inp = synth.make_inputs(cfg, seed=13)
    out = oracle_mod.run_frame(cfg, w, inp, keep_kv=True)
    for r in range(cfg.rows):
        z, ks, vs = _hf_frame(cfg, w, inp, r, out["codes"][r])
        assert np.abs(out["logits"][r] - z).max() <= 2e-6 * max(1.0, np.abs(z).max())
        k_or = out["k_cache"][:, r].transpose(0, 2, 1, 3)
        v_or = out["v_cache"][:, r].transpose(0, 2, 1, 3)
        assert np.abs(k_or - ks).max() <= 2e-6 * max(1.0, np.abs(ks).max())
        assert np.abs(v_or - vs).max() <= 2e-6 * max(1.0, np.abs(vs).max())
    # the variant changes the frame (it is not silently ignored)
    plain = oracle_mod.run_frame(cfg.with_(qk_norm=False), w, inp, forced_codes=out["codes"])
    assert np.abs(plain["logits"] - out["logits"]).max() > 1e-3


def test_oracle_qk_norm_is_per_head_and_scale_free(oracle_mod):
    """RMSNorm of a head makes it independent of that head's scale: scaling
    the W_q rows of one q head, or the W_k rows of one k head, by 3 leaves
    the logits unchanged to fp32 rounding, while the same scaling without
    the norm changes them.  Scaling every row of the q block by a different
    factor per head also leaves them unchanged (a norm over all heads at once
    would not)."""
    cfg = TINY.with_(rows=2, qk_norm=True, n_positions=4)
    w = synth.make_weights(cfg, seed=17, gain_jitter=True)
    inp = synth.make_inputs(cfg, seed=17)
    base = oracle_mod.run_frame(cfg, w, inp)
    d, qd = cfg.head_dim, cfg.n_q_heads * cfg.head_dim
    for rows_sl, fac in ((slice(0, d), 3.0), (slice(qd + d, qd + 2 * d), 3.0), (None, None)):
        w2 = dict(w)
        for l in range(cfg.n_layers):
            m = w[f"w_qkv.{l}"].copy()
            if rows_sl is None:
                for h in range(cfg.n_q_heads):
                    m[h * d:(h + 1) * d] *= np.float32(0.5 + h)
            else:
                m[rows_sl] *= np.float32(fac)
            w2[f"w_qkv.{l}"] = m
        alt = oracle_mod.run_frame(cfg, w2, inp, forced_codes=base["codes"])
        assert np.abs(alt["logits"] - base["logits"]).max() <= 1e-5 * np.abs(base["logits"]).max()
        off = oracle_mod.run_frame(cfg.with_(qk_norm=False), w2, inp, forced_codes=base["codes"])
        ref = oracle_mod.run_frame(cfg.with_(qk_norm=False), w, inp, forced_codes=base["codes"])
        assert np.abs(off["logits"] - ref["logits"]).max() > 1e-4


def test_oracle_bf16_close_to_fp64_stack(oracle_mod):
    """bf16 rounding at the storage points moves logits by a bf16-sized amount only."""
    cfg = TINY.with_(rows=2, dtype="bf16")
    w = synth.make_weights(cfg, seed=5)
    inp = synth.make_inputs(cfg, seed=5)
    out = oracle_mod.run_frame(cfg, w, inp, keep_kv=True)
    for r in range(cfg.rows):
        z, ks, _ = _hf_frame(cfg, w, inp, r, out["codes"][r])
        err = np.abs(out["logits"][r] - z).max()
        assert err < 0.05, err
        assert err > 0.0  # the rounding points are actually applied
    # every stored K/V value is a bf16 value
    kb = out["k_cache"].view(np.uint32)
    assert not np.any(kb & 0xFFFF)


# ------------------------------------------------------------------ frame wiring

def test_causality_and_head_wiring(oracle_mod):
    """Code j only reaches positions after j: forcing a different c_j leaves
    logits 1..j bitwise unchanged and changes logits j+1."""
    cfg = TINY.with_(rows=1, n_positions=5)
    w = synth.make_weights(cfg, seed=3)
    inp = synth.make_inputs(cfg, seed=3)
    base = oracle_mod.run_frame(cfg, w, inp)
    for j in range(1, cfg.n_positions - 1):
        forced = base["codes"].copy()
        forced[0, j - 1] = (forced[0, j - 1] + 7) % cfg.vocab
        alt = oracle_mod.run_frame(cfg, w, inp, forced_codes=forced)
        assert np.array_equal(alt["logits"][0, :j], base["logits"][0, :j])
        assert not np.array_equal(alt["logits"][0, j], base["logits"][0, j])
        assert np.array_equal(alt["codes"][0, :j], base["codes"][0, :j])


def test_embedding_sum_is_exact_ordered_float_sum(oracle_mod):
    for cfg in (TINY.with_(rows=4), TINY.with_(rows=4, dtype="bf16")):
        w = synth.make_weights(cfg, seed=2)
        inp = synth.make_inputs(cfg, seed=2)
        out = oracle_mod.run_frame(cfg, w, inp)
        for r in range(cfg.rows):
            codes = [int(inp["code0"][r])] + list(out["codes"][r])
            s = synth.as_f32(cfg, w["embed.0"])[codes[0]].copy()
            for j in range(1, cfg.n_positions):
                s = (s + synth.as_f32(cfg, w[f"embed.{j}"])[codes[j]]).astype(np.float32)
            assert np.array_equal(s, out["embsum"][r])


def test_input_projection_identity_and_thread_count(oracle_mod):
    """W_in = I makes position 0 the input itself (same logits as feeding x);
    the thread count never changes a result."""
    cfg = TINY.with_(rows=5)
    w = synth.make_weights(cfg, seed=4)
    inp = synth.make_inputs(cfg, seed=4)
    a = oracle_mod.run_frame(cfg, w, inp, n_threads=1)
    b = oracle_mod.run_frame(cfg, w, inp, n_threads=7)
    for k in ("codes", "embsum", "logits"):
        assert np.array_equal(a[k], b[k])
    w2 = dict(w)
    w2["w_in"] = np.eye(cfg.hidden, dtype=np.float32)
    out = oracle_mod.run_frame(cfg, w2, inp, keep_hidden=True)
    z, _, _ = _hf_frame(cfg, w2, inp, 0, out["codes"][0])
    assert np.abs(out["logits"][0] - z).max() < 2e-6


def test_subset_rows_match_full_batch(oracle_mod):
    cfg = TINY.with_(rows=6)
    w = synth.make_weights(cfg, seed=9)
    inp = synth.make_inputs(cfg, seed=9)
    full = oracle_mod.run_frame(cfg, w, inp)
    sub = oracle_mod.run_frame(cfg, w, inp, rows=[4, 1])
    assert np.array_equal(sub["logits"], full["logits"][[4, 1]])
    assert np.array_equal(sub["codes"], full["codes"][[4, 1]])


def test_offsets_advance_once_per_draw(oracle_mod):
    cfg = TINY.with_(rows=3, sampled=True)
    w = synth.make_weights(cfg, seed=1)
    inp = synth.make_inputs(cfg, seed=1)
    out = oracle_mod.run_frame(cfg, w, inp)
    assert np.array_equal(out["offset"], inp["offset"] + np.uint64(cfg.n_positions - 1))


def test_sampled_frame_equals_single_draws(oracle_mod):
    """Each sampled code is the single draw from that position's logits at
    offset + (j - 1) (section "Testing": fused draws equal single sample calls)."""
    cfg = TINY.with_(rows=3, sampled=True)
    w = synth.make_weights(cfg, seed=8)
    inp = synth.make_inputs(cfg, seed=8)
    out = oracle_mod.run_frame(cfg, w, inp)
    for r in range(cfg.rows):
        for j in range(1, cfg.n_positions):
            c, _ = oracle_mod.draw(out["logits"][r, j - 1], inp["temperature"][r], inp["top_k"][r],
                                   inp["top_p"][r], int(inp["seed"][r]),
                                   int(inp["offset"][r]) + j - 1)
            assert c == out["codes"][r, j - 1]


# ------------------------------------------------------------------ philox / rounding

def test_philox4x64_matches_numpy(oracle_mod):
    rng = np.random.default_rng(0)
    cases = [(np.array([1, 0, 0, 0], np.uint64), np.array([0, 0], np.uint64)),
             (np.array([0, 1, 0, 0], np.uint64), np.array([2**64 - 1, 2**64 - 1], np.uint64))]
    for _ in range(64):
        cases.append((rng.integers(0, 2**64, 4, dtype=np.uint64) | np.uint64(1),
                      rng.integers(0, 2**64, 2, dtype=np.uint64)))
    for ctr, key in cases:
        # numpy's Philox adds one (with carry) to its 256-bit counter before each block
        v = sum(int(c) << (64 * i) for i, c in enumerate(ctr)) - 1
        prev = np.array([(v >> (64 * i)) & (2**64 - 1) for i in range(4)], np.uint64)
        ref = np.random.Philox(counter=prev, key=key).random_raw(4)
        assert np.array_equal(oracle_mod.philox4x64(ctr, key), ref)


def test_bf16_rounding_matches_torch(oracle_mod):
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                           # exact halfway cases (both parities) and near-halfway neighbours
                           (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                           (np.arange(1, 200, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
                           np.array([0.0, -0.0, 1e-40, 3.0e38], np.float32)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle_mod.round_bf16(v) for v in vals], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ draw

def test_greedy_planted_and_ties(oracle_mod):
    z = np.zeros(64, np.float32)
    z[37] = 5.0
    assert oracle_mod.draw(z)[0] == 37
    z[12] = 5.0
    assert oracle_mod.draw(z)[0] == 12          # lowest index on a tie
    code, m = oracle_mod.draw(z)
    assert m[0] == 0.0
    z[12] = 4.5
    code, m = oracle_mod.draw(z)
    assert code == 37 and m[0] == pytest.approx(0.5)


def _check_kept_definition(z, T, k, p, kept):
    y = (z / np.float32(T)).astype(np.float32)
    V = len(z)
    kk = V if (k <= 0 or k >= V) else k
    assert 1 <= len(kept) <= kk
    rest = np.setdiff1d(np.arange(V), kept)
    if len(rest):
        assert y[kept].min() >= y[rest].max()      # a top set
    top = np.argsort(-y.astype(np.float64), kind="stable")[:kk]
    e = np.exp(y[top].astype(np.float64) - y[top].max())
    prob = dict(zip(top.tolist(), (e / e.sum()).tolist()))
    mass = sum(prob[i] for i in kept)
    if p < 1.0:
        assert mass >= p - 1e-12 or len(kept) == kk
        smallest = min(kept, key=lambda i: (y[i], -i))
        assert mass - prob[smallest] < p           # no shorter prefix reaches p
    else:
        assert len(kept) == kk


def test_kept_set_definition_bruteforce(oracle_mod):
    rng = np.random.default_rng(2)
    for _ in range(300):
        V = int(rng.integers(2, 17))
        z = rng.standard_normal(V).astype(np.float32) * np.float32(rng.uniform(0.2, 3))
        T = float(rng.uniform(0.3, 1.5))
        k = int(rng.choice([0, 1, 2, 3, 5, V, V + 3]))
        p = float(rng.choice([0.3, 0.5, 0.8, 0.95, 1.0]))
        kept = oracle_mod.kept_set(z, T, k, p)
        _check_kept_definition(z, T, k, p, kept)
        code, _ = oracle_mod.draw(z, T, k, p, seed=int(rng.integers(0, 2**63)), counter=3)
        assert code in kept


def test_degenerate_sampling_is_greedy(oracle_mod):
    rng = np.random.default_rng(3)
    for i in range(50):
        z = rng.standard_normal(200).astype(np.float32)
        g = int(np.argmax(z))
        assert oracle_mod.draw(z, 0.9, 1, 0.9, seed=i, counter=i)[0] == g   # top-k 1
        assert oracle_mod.draw(z, 0.9, 0, 0.0, seed=i, counter=i)[0] == g   # top-p 0
        assert oracle_mod.draw(z, 0.0, 50, 0.9, seed=i, counter=i)[0] == g  # T <= 0


def test_gumbel_max_law_chi_square(oracle_mod):
    """Codes drawn over many counters follow the renormalised kept distribution."""
    from scipy.stats import chisquare
    z = np.array([2.0, 1.5, 1.4, 0.3, 0.2, -1.0, 0.9, 1.1, -0.5, 0.0, 1.45, -2.0], np.float32)
    for T, k, p in [(1.0, 0, 1.0), (0.7, 6, 1.0), (1.2, 0, 0.8), (0.9, 8, 0.9)]:
        kept = oracle_mod.kept_set(z, T, k, p)
        y = (z / np.float32(T)).astype(np.float64)
        pr = np.exp(y[kept] - y[kept].max())
        pr /= pr.sum()
        n = 6000
        counts = np.zeros(len(z), np.int64)
        for c in range(n):
            counts[oracle_mod.draw(z, T, k, p, seed=12345, counter=c)[0]] += 1
        assert counts[np.setdiff1d(np.arange(len(z)), kept)].sum() == 0
        stat = chisquare(counts[kept], pr * n)
        assert stat.pvalue > 1e-4, (T, k, p, stat)


def test_draw_margins(oracle_mod):
    z = np.linspace(-1, 1, 32).astype(np.float32)
    code, m = oracle_mod.draw(z, 1.0, 5, 1.0, seed=1, counter=2)
    y = np.sort(z)[::-1]
    assert m[1] == pytest.approx(float(y[4] - y[5]), abs=1e-6)
    assert np.isinf(m[2]) and np.isinf(m[3])
    code, m = oracle_mod.draw(z, 1.0, 0, 0.5, seed=1, counter=2)
    assert m[2] > 0 and m[3] >= 0


# ------------------------------------------------------------------ numbers the pages print

def test_page_counts_and_byte_model():
    """Structural numbers printed by the pages (tests/golden/page_counts.json)."""
    g = json.load(open(os.path.join(GOLDEN, "page_counts.json")))
    cfg = synth.CONFIGS["l5_r64"]
    L, P = cfg.n_layers, cfg.n_positions
    assert 5 * L * P + 1 + (P - 1) + P == g["phases_per_frame"]
    assert L * P == g["loop_attention_launches"]
    assert P - 1 == g["loop_sampling_launches"] == g["loop_embedding_launches"]
    layer_set = L * cfg.layer_weight_bytes()
    assert abs(layer_set / 1e6 - g["layer_weights_MB"]) < 0.5
    assert abs(cfg.frame_weight_bytes() / 1e9 - g["frame_bytes_GB"]) < 0.05
    floor_ms = cfg.frame_weight_bytes() / (g["h200_hbm_TBps"] * 1e12) * 1e3
    assert abs(floor_ms - g["floor_ms"]) < 0.005
