"""Pins for the oracle's forward pass (CPU only).

The decoder is the Qwen3 family of "Model-agnostic LLM inference", section
"Supported models": grouped-query attention with RMSNorm on Q/K, RoPE, a
SiLU-gated feed-forward block, tied embeddings, no attention bias.  Greedy
decoding takes the arg-max each step ("Model-agnostic LLM inference", section
"Notes").  Nothing here compares the oracle with itself: each test checks it
against an independent brute force, a closed form, or an invariant of the maths.
"""
import dataclasses

import numpy as np
import pytest

from oracle import Oracle, quantize_model, quantize_rows, bf16
from workloads import SHAPES, ModelShape, make_weights, make_prompt
import reference_f64 as ref

TINY = SHAPES["tiny"]
# head_dim * heads != hidden (as in Qwen3-0.6B), so a transposed projection or a
# 1/sqrt(hidden/heads) attention scale cannot pass unnoticed
WIDE = ModelShape(hidden=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=64,
                  intermediate=256, vocab=512)


def _setup(shape, seed=0, gains="ones"):
    w = make_weights(shape, seed=seed, gains=gains)
    return w, quantize_model(w)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b))


@pytest.mark.parametrize("shape,gains", [(TINY, "ones"), (TINY, "uniform"), (WIDE, "uniform")])
def test_exact_mode_matches_bruteforce(shape, gains):
    _, qm = _setup(shape, gains=gains)
    W = ref.dequantized(qm)
    prompt = make_prompt(shape.vocab, 16, 1000)
    orc = Oracle(shape, qm, mode="exact")
    out = orc.generate(prompt, 8)
    ids_ref, logits_ref = ref.greedy(shape, W, prompt, 8)
    np.testing.assert_array_equal(out["ids"], ids_ref)
    assert _rel(out["logits"], logits_ref) < 1e-10


@pytest.mark.parametrize("shape,gains", [(TINY, "ones"), (WIDE, "uniform")])
def test_bf16_mode_stays_near_exact_bruteforce(shape, gains):
    """bf16 rounding of every activation moves the logits only by accumulated rounding.

    Each path through the 2-layer model crosses about a dozen bf16 rounding points of
    at most 2^-9 relative error each; the measured max-abs logit gap is 2-3.5% of the
    logit RMS over 3 seeds, so 6e-2 bounds it.  Greedy ids must agree wherever the
    oracle's top-1/top-2 margin exceeds 5e-2.
    """
    _, qm = _setup(shape, gains=gains)
    W = ref.dequantized(qm)
    prompt = make_prompt(shape.vocab, 16, 1000)
    orc = Oracle(shape, qm, mode="bf16")
    out = orc.generate(prompt, 16)
    seq = np.concatenate([prompt, out["ids"][:-1]])
    lg = ref.logits_all(shape, W, seq)[len(prompt) - 1:]
    for k in range(16):
        rms = np.sqrt(np.mean(lg[k] ** 2))
        assert np.max(np.abs(out["logits"][k] - lg[k])) / rms <= 6e-2
        if out["margin"][k] > 5e-2:
            assert out["ids"][k] == int(np.argmax(lg[k]))


def test_bruteforce_matches_transformers_qwen3():
    """The brute force agrees with the transformers Qwen3 implementation (run, not copied)."""
    transformers = pytest.importorskip("transformers")
    torch = pytest.importorskip("torch")
    from transformers import Qwen3Config, Qwen3ForCausalLM
    shape = WIDE
    _, qm = _setup(shape, gains="uniform")
    W = ref.dequantized(qm)
    cfg = Qwen3Config(vocab_size=shape.vocab, hidden_size=shape.hidden,
                      intermediate_size=shape.intermediate, num_hidden_layers=shape.n_layers,
                      num_attention_heads=shape.n_heads, num_key_value_heads=shape.n_kv_heads,
                      head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps,
                      rope_theta=shape.rope_theta, tie_word_embeddings=True,
                      attention_bias=False, max_position_embeddings=256,
                      attn_implementation="eager")
    try:
        cfg.rope_parameters = {"rope_type": "default", "rope_theta": shape.rope_theta}
    except Exception:
        pass
    model = Qwen3ForCausalLM(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    sd = {"model.embed_tokens.weight": t(W["embed"]), "model.norm.weight": t(W["final_norm"])}
    hf = {"q": "self_attn.q_proj", "k": "self_attn.k_proj", "v": "self_attn.v_proj",
          "o": "self_attn.o_proj", "gate": "mlp.gate_proj", "up": "mlp.up_proj",
          "down": "mlp.down_proj", "q_norm": "self_attn.q_norm", "k_norm": "self_attn.k_norm",
          "in_norm": "input_layernorm", "post_norm": "post_attention_layernorm"}
    for i, L in enumerate(W["layers"]):
        for k, name in hf.items():
            sd[f"model.layers.{i}.{name}.weight"] = t(L[k])
    sd["lm_head.weight"] = t(W["embed"])
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not [m for m in missing if "rotary" not in m], missing
    ids = make_prompt(shape.vocab, 24, 1001)
    with torch.no_grad():
        got = model(torch.from_numpy(ids.astype(np.int64))[None]).logits[0].numpy()
    want = ref.logits_all(shape, W, ids)
    # transformers computes RMSNorm and the RoPE tables in fp32, hence 1e-4
    assert _rel(got, want) < 1e-4


def test_rope_position_zero_is_identity_and_rotation_preserves_norm():
    _, qm = _setup(TINY)
    orc = Oracle(TINY, qm, mode="exact")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 4, TINY.head_dim))
    np.testing.assert_array_equal(orc.rope(x, np.zeros(3, dtype=int)), x)
    y = orc.rope(x, np.array([1, 17, 400]))
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # relative position: <R_p a, R_q b> depends on p - q only
    a, b = x[0, 0], x[1, 0]
    d1 = orc.rope(a[None, None], [10])[0, 0] @ orc.rope(b[None, None], [3])[0, 0]
    d2 = orc.rope(a[None, None], [107])[0, 0] @ orc.rope(b[None, None], [100])[0, 0]
    assert abs(d1 - d2) < 1e-12
    orc16 = Oracle(TINY, qm, mode="bf16")
    xb = bf16(x)
    np.testing.assert_array_equal(orc16.rope(xb, np.zeros(3, dtype=int)), xb)


def test_attention_closed_forms():
    _, qm = _setup(TINY)
    orc = Oracle(TINY, qm, mode="exact")
    rng = np.random.default_rng(6)
    KV, H, D = TINY.n_kv_heads, TINY.n_heads, TINY.head_dim
    K = rng.standard_normal((KV, 9, D))
    V = rng.standard_normal((KV, 9, D))
    q = rng.standard_normal((1, H, D))
    # a single position: the output is that position's value row
    o = orc.attention(q, K[:, :1], V[:, :1], [0])
    for h in range(H):
        np.testing.assert_array_equal(o[0, h], V[h // (H // KV), 0])
    # zero query: uniform weights, the output is the mean of the visible values
    o = orc.attention(np.zeros((1, H, D)), K, V, [8])
    for h in range(H):
        np.testing.assert_allclose(o[0, h], V[h // (H // KV)].mean(axis=0), rtol=1e-13, atol=1e-15)
    # row r sees positions 0..r only
    o_all = orc.attention(np.repeat(q, 9, 0), K, V, np.arange(9))
    o_3 = orc.attention(q, K[:, :4], V[:, :4], [3])
    np.testing.assert_allclose(o_all[3], o_3[0], rtol=1e-13)


def test_causality_appending_tokens_leaves_earlier_logits():
    _, qm = _setup(TINY)
    for mode in ("exact", "bf16"):
        orc = Oracle(TINY, qm, mode=mode)
        ids = make_prompt(TINY.vocab, 20, 1002)
        s1 = orc.new_sequence()
        full = orc.forward(s1, ids, logits_rows="all")
        s2 = orc.new_sequence()
        part = orc.forward(s2, ids[:12], logits_rows="all")
        tol = 1e-12 if mode == "exact" else 2e-2
        assert _rel(full[:12], part) <= tol


def test_prefill_equals_stepwise_decode():
    _, qm = _setup(WIDE, gains="uniform")
    orc = Oracle(WIDE, qm, mode="exact")
    ids = make_prompt(WIDE.vocab, 12, 1003)
    s1 = orc.new_sequence()
    block = orc.forward(s1, ids, logits_rows="all")
    s2 = orc.new_sequence()
    steps = np.stack([orc.forward(s2, [t]) for t in ids])
    assert _rel(block, steps) < 1e-12


def test_gqa_equals_mha_with_duplicated_kv_heads():
    """Duplicating each KV head for its query heads turns GQA into MHA; outputs agree."""
    shape = WIDE
    w, qm = _setup(shape, gains="uniform")
    G = shape.n_heads // shape.n_kv_heads
    D = shape.head_dim
    mha_shape = dataclasses.replace(shape, n_kv_heads=shape.n_heads)
    qm2 = {"embed": qm["embed"], "final_norm": qm["final_norm"], "layers": []}
    for L in qm["layers"]:
        L2 = dict(L)
        for m in ("k", "v"):
            q8, s = L[m]
            rows = np.concatenate([np.arange(g * D, (g + 1) * D)
                                   for g in range(shape.n_kv_heads) for _ in range(G)])
            L2[m] = (q8[rows], s[rows])
        qm2["layers"].append(L2)
    ids = make_prompt(shape.vocab, 10, 1004)
    a = Oracle(shape, qm, mode="exact").generate(ids, 4)
    b = Oracle(mha_shape, qm2, mode="exact").generate(ids, 4)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    assert _rel(a["logits"], b["logits"]) < 1e-12


def test_bigram_closed_form_when_blocks_write_nothing():
    """With o_proj = down_proj = 0 both residual blocks add zero, so the logits at any
    position are RMSNorm(embedding row of the current token) times the tied embedding."""
    w, _ = _setup(TINY, gains="uniform")
    for L in w["layers"]:
        L["o"] = np.zeros_like(L["o"])
        L["down"] = np.zeros_like(L["down"])
    qm = quantize_model(w)
    Eq, Es = qm["embed"]
    g = qm["final_norm"].astype(np.float64)
    eps = TINY.rms_eps
    ids = make_prompt(TINY.vocab, 10, 1005)
    orc = Oracle(TINY, qm, mode="bf16")
    got = orc.forward(orc.new_sequence(), ids, logits_rows="all")
    for r, t in enumerate(ids):
        e = bf16(Eq[t].astype(np.float32) * Es[t])
        f = bf16(e / np.sqrt(np.mean(e * e) + eps) * g)
        want = np.array([np.float32(np.dot(Eq[v].astype(np.float64), f) * float(Es[v]))
                         for v in range(TINY.vocab)])
        np.testing.assert_allclose(got[r], want, rtol=1e-6, atol=1e-7)


def test_zero_matrix_rows_quantize_to_zero():
    q, s = quantize_rows(np.zeros((3, 8), np.float32))
    assert np.all(q == 0) and np.all(s == 0)


# ---- the pins are sensitive: plant plausible mistakes in a copy of the oracle ------------

class _Interleaved(Oracle):
    def rope(self, x, positions):
        ang = np.asarray(positions, np.float64)[:, None] * self.inv_freq[None, :]
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        a, b = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
        return self._act(out)


class _HiddenScale(Oracle):
    def attention(self, q, K, V, positions):
        D = self.shape.head_dim
        ratio = np.sqrt(D) / np.sqrt(self.shape.hidden / self.shape.n_heads)
        return super().attention(q * ratio, K, V, positions)


class _ModuloHeadMap(Oracle):
    def attention(self, q, K, V, positions):
        H, KV = self.shape.n_heads, self.shape.n_kv_heads
        perm = [h for g in range(KV) for h in range(H) if h % KV == g]
        inv = np.argsort(perm)
        return super().attention(q[:, perm], K, V, positions)[:, inv]


class _NoQKGain(Oracle):
    def rmsnorm(self, y, g):
        if y.ndim == 3:
            g = np.ones_like(g)
        return super().rmsnorm(y, g)


@pytest.mark.parametrize("bad", [_Interleaved, _HiddenScale, _ModuloHeadMap, _NoQKGain])
def test_planted_mistakes_fail_the_bruteforce_pin(bad):
    shape = WIDE
    _, qm = _setup(shape, gains="uniform")
    W = ref.dequantized(qm)
    prompt = make_prompt(shape.vocab, 12, 1006)
    got = bad(shape, qm, mode="exact").forward(Oracle(shape, qm).new_sequence(), prompt,
                                              logits_rows="all")
    want = ref.logits_all(shape, W, prompt)
    assert _rel(got, want) > 1e-3
