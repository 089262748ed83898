"""Bar-free exact checks of the decode-step kernels at the Qwen3-0.6B shape (GPU).

Integer-valued weights whose every row reaches +-127 quantize to themselves with scale
exactly 1 (absmax / 127 = 1, "Model-agnostic LLM inference", section "The quantized load
cache": int8 codes with one scale per row).  With integer-valued bf16 activations of
magnitude <= 8, every dot product is an integer below 2^24, so fp32 accumulation is exact
in any order and each kernel's output is fixed to the bit: bf16(acc) for q|k|v, bf16(x +
bf16(acc)) for the residual projections, SiLU(bf16(g)) * bf16(u) rounded once for the
gated feed-forward, and the fp32 logits themselves for the LM head.  Rows that enter an
RMSNorm have one magnitude c in every element, so the normalized row is sign(x) times
the gain to the bit (x / rms(x) is within a few ulps of +-1, and the gains are small
integers that bf16 rounding then restores exactly).

Each check runs the kernel class exactly as a decode step launches it at that batch
(qd_run_op): B = 1 (register GEMV), 2 and 16 (MFMA skinny tiles of 16 rows), 17 and 32 (two
16-row tiles, residual projections split over K across work-groups), and the LM head's
full 151,936-row sweep with its fused arg-max (greedy decoding is the arg-max, lowest
index among equal maxima; "Model-agnostic LLM inference", section "Notes").
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bf16
from workloads import SHAPES
from parity import say

pytestmark = pytest.mark.gpu

SH = dataclasses.replace(SHAPES["qwen3-0.6b"], n_layers=1)
D_, H_, KV_, HD_ = SH.head_dim, SH.n_heads, SH.n_kv_heads, SH.head_dim * SH.n_heads
NQKV = HD_ + 2 * KV_ * D_
BATCHES = [1, 2, 16, 17, 32]
GATE_SIGN_K = SH.hidden // 2   # the gate rows' dominant half (see _integer_weights)


def _int_rows(rng, rows, cols, lim=127):
    """Integer-valued fp32 rows in [-lim, lim], each holding +-127 once (scale exactly 1)."""
    w = rng.integers(-lim, lim + 1, (rows, cols)).astype(np.float32)
    w[np.arange(rows), rng.integers(0, cols, rows)] = np.where(rng.random(rows) < 0.5, -127, 127)
    return w


PLANT_LO = 1000 + 37 * np.arange(32)            # planted arg-max rows, one pair per batch row
PLANT_HI = SH.vocab - 1 - 3 * np.arange(32)


def _integer_weights(seed=21):
    """Integer weights for the op checks.  The gate rows put +-127 (one sign per row) on a
    shared sign pattern over the first half of k and -1..1 elsewhere, so every gate
    accumulator is at least 127*512 - 8*512 in magnitude: SiLU is then exactly the identity
    (e^-g underflows against 1) or exactly zero (e^-g overflows), with no rounding of a
    transcendental left to disagree about.  The embedding rows are +-127 sign patterns;
    rows PLANT_LO[b] and PLANT_HI[b] hold the same pattern P_b, the LM-head maximum for an
    input row with the signs of P_b."""
    rng = np.random.default_rng(seed)
    d, I, V = SH.hidden, SH.intermediate, SH.vocab
    w = {"embed": np.where(rng.random((V, d)) < 0.5, -127.0, 127.0).astype(np.float32)}
    plant = np.where(rng.random((32, d)) < 0.5, -1.0, 1.0)
    w["embed"][PLANT_LO] = 127.0 * plant
    w["embed"][PLANT_HI] = 127.0 * plant
    L = {"q": _int_rows(rng, HD_, d), "k": _int_rows(rng, KV_ * D_, d),
         "v": _int_rows(rng, KV_ * D_, d), "o": _int_rows(rng, d, HD_),
         "up": _int_rows(rng, I, d), "down": _int_rows(rng, d, I)}
    sigma = np.where(rng.random(GATE_SIGN_K) < 0.5, -1.0, 1.0)
    t = np.where(rng.random(I) < 0.5, -1.0, 1.0)
    gate = rng.integers(-1, 2, (I, d)).astype(np.float32)
    gate[:, :GATE_SIGN_K] = (127.0 * t[:, None] * sigma[None, :]).astype(np.float32)
    L["gate"] = gate
    L["in_norm"] = rng.integers(1, 9, d).astype(np.float32)
    L["post_norm"] = rng.integers(1, 9, d).astype(np.float32)
    L["q_norm"] = np.ones(D_, np.float32)
    L["k_norm"] = np.ones(D_, np.float32)
    w["layers"] = [L]
    w["final_norm"] = rng.integers(1, 9, d).astype(np.float32)
    return w, {"sigma": sigma, "plant": plant}


@pytest.fixture(scope="module")
def exact_model():
    import int8_weight_only_amd as qd
    w, aux = _integer_weights()
    say("[gpu] exact: loading the integer-weight model at the Qwen3-0.6B shape (1 layer)")
    m = qd.Model(SH, w, max_batch=32, max_ctx=64, max_prefill_tokens=64)
    yield m, w, aux
    m.close()


def _bf(a):
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16).cuda()


def _vals(t):
    return t.float().cpu().numpy().astype(np.float64)


def _norm_input(rng, B, sign_prefix=None):
    """Rows of one magnitude c_b (1..5) with random signs; returns (x, signs)."""
    s = np.where(rng.random((B, SH.hidden)) < 0.5, -1.0, 1.0)
    if sign_prefix is not None:
        s[:, :sign_prefix.size] = sign_prefix
    c = (np.arange(B) % 5 + 1).astype(np.float64)[:, None]
    return c * s, s


def test_quantized_codes_are_the_integers(exact_model):
    m, w, _ = exact_model
    for t in ("embed",):
        q, s = m.export_quantized(t)
        assert np.all(s == 1.0) and np.array_equal(q, w[t].astype(np.int8))
    for t in ("q", "o", "gate", "down"):
        q, s = m.export_quantized(t, 0)
        assert np.all(s == 1.0) and np.array_equal(q, w["layers"][0][t].astype(np.int8)), t


@pytest.mark.parametrize("B", BATCHES)
def test_embedding_rows_bit_exact(exact_model, B):
    m, w, _ = exact_model
    ids = np.random.default_rng(B).integers(0, SH.vocab, B).astype(np.int32)
    ids[0], ids[-1] = 0, SH.vocab - 1
    out = m.run_op("embed", torch.as_tensor(ids).cuda())
    np.testing.assert_array_equal(_vals(out), w["embed"][ids].astype(np.float64))


# the batched folded-norm kernels load the activation rows contiguously and reorder them
# in LDS (default, above 8 rows) or load them in the matrix-core operand layout
XSTAGE = pytest.mark.parametrize("xstage", [1, 0], ids=["row-staged", "operand-loads"])


def _run_op_xstage(m, op, x, xstage):
    m.set_tuning(skinny_xstage=xstage)
    try:
        return m.run_op(op, x)
    finally:
        m.set_tuning(skinny_xstage=1)


@XSTAGE
@pytest.mark.parametrize("B", BATCHES)
def test_qkv_projection_bit_exact(exact_model, B, xstage):
    m, w, _ = exact_model
    L = w["layers"][0]
    x, s = _norm_input(np.random.default_rng(100 + B), B)
    h = s * L["in_norm"].astype(np.float64)                  # RMSNorm(x, gain), exactly
    W = np.concatenate([L["q"], L["k"], L["v"]]).astype(np.float64)
    want = bf16(h @ W.T)
    got = _vals(_run_op_xstage(m, "qkv", _bf(x), xstage))
    assert np.max(np.abs(h @ W.T)) < 2 ** 24
    np.testing.assert_array_equal(got, want, err_msg=f"B={B}")
    say(f"[gpu] exact q|k|v B={B}: {got.size} outputs bit-exact")


@XSTAGE
@pytest.mark.parametrize("B", BATCHES)
def test_gate_up_silu_bit_exact(exact_model, B, xstage):
    m, w, aux = exact_model
    L = w["layers"][0]
    x, s = _norm_input(np.random.default_rng(200 + B), B, sign_prefix=aux["sigma"])
    h = s * L["post_norm"].astype(np.float64)
    g = bf16(h @ L["gate"].astype(np.float64).T).astype(np.float32)
    u = bf16(h @ L["up"].astype(np.float64).T).astype(np.float32)
    assert np.min(np.abs(g)) > 127 * GATE_SIGN_K - 8 * SH.hidden
    with np.errstate(over="ignore"):
        silu = (g / (np.float32(1) + np.exp(-g))).astype(np.float32)
    want = bf16((silu * u).astype(np.float32))
    got = _vals(_run_op_xstage(m, "gateup", _bf(x), xstage))
    np.testing.assert_array_equal(got, want, err_msg=f"B={B}")
    say(f"[gpu] exact gate/up B={B}: {got.size} outputs bit-exact, "
        f"{int(np.sum(want != 0))} through the identity branch")


@pytest.mark.parametrize("op,K", [("o", HD_), ("down", SH.intermediate)])
@pytest.mark.parametrize("B", BATCHES)
def test_residual_projections_bit_exact(exact_model, op, K, B):
    m, w, _ = exact_model
    rng = np.random.default_rng(300 + B + K)
    a = rng.integers(-8, 9, (B, K)).astype(np.float64)
    resid = rng.integers(-100, 101, (B, SH.hidden)).astype(np.float64)
    W = w["layers"][0][op].astype(np.float64)
    acc = a @ W.T
    assert np.max(np.abs(acc)) < 2 ** 24
    want = bf16(resid + bf16(acc))
    got = _vals(m.run_op(op, _bf(a), resid=_bf(resid)))
    np.testing.assert_array_equal(got, want, err_msg=f"{op} B={B}")


@pytest.mark.parametrize("B", BATCHES)
def test_lm_head_logits_and_planted_ties_bit_exact(exact_model, B):
    """Every row's maximum sits at two planted indices far apart in the 151,936-row sweep
    (so in different work-groups' row blocks): the fused arg-max must return the lower."""
    m, w, aux = exact_model
    s = aux["plant"][:B]
    x = (np.arange(B) % 5 + 1).astype(np.float64)[:, None] * s
    f = s * w["final_norm"].astype(np.float64)
    want = f @ w["embed"].astype(np.float64).T
    assert np.all(np.argmax(want, axis=1) == PLANT_LO[:B])
    got, ids = m.run_op("lmhead", _bf(x))
    got = got.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(ids.cpu().numpy(), PLANT_LO[:B])
    say(f"[gpu] exact LM head B={B}: {got.size} logits bit-exact, planted ties to the lower index")


@pytest.fixture(scope="module")
def bigram_model():
    """o_proj = down_proj = 0: every layer adds exactly zero to the residual, so the logits
    of a fed token t are E . (sign(E[t]) * g_final) whatever the context -- integers, exact in
    fp32.  Each fed token's row is duplicated at a lower index, which must win the arg-max."""
    import int8_weight_only_amd as qd
    w, _ = _integer_weights(seed=22)
    L = w["layers"][0]
    L["o"] = np.zeros_like(L["o"])
    L["down"] = np.zeros_like(L["down"])
    rng = np.random.default_rng(23)
    fed = rng.choice(np.arange(20000, 150000), size=96, replace=False).astype(np.int32)
    dup = rng.choice(np.arange(3000, 20000), size=96, replace=False).astype(np.int32)
    w["embed"][dup] = w["embed"][fed]
    say("[gpu] exact: loading the zero-o/down integer model (Qwen3-0.6B shape, 1 layer)")
    m = qd.Model(SH, w, max_batch=32, max_ctx=64, max_prefill_tokens=128)
    yield m, w, fed, dup
    m.close()


def _bigram_logits(w, t):
    E = w["embed"].astype(np.float64)
    f = np.sign(E[t]) * w["final_norm"].astype(np.float64)
    return f @ E.T


def test_bigram_single_stream_through_the_c_abi(bigram_model):
    """qd_prefill (last row of a 3-token prompt) and three qd_decode_step calls at B=1."""
    m, w, fed, dup = bigram_model
    nxt, lg = m.prefill([fed[:3]], logits=True)
    torch.cuda.synchronize()
    steps = [(lg, nxt, 2)]
    for k in range(3, 6):
        nxt, lg = m.decode_step(torch.tensor([fed[k]], dtype=torch.int32, device="cuda"), logits=True)
        torch.cuda.synchronize()
        steps.append((lg, nxt, k))
    for lg, nxt, k in steps:
        np.testing.assert_array_equal(lg[0].cpu().numpy().astype(np.float64),
                                      _bigram_logits(w, fed[k]), err_msg=f"token {k}")
        assert int(nxt[0].item()) == int(dup[k]), (k, int(nxt[0].item()), int(dup[k]))
    say("[gpu] exact bigram B=1: prefill row + 3 decode steps, 151,936 logits bit-exact each")


def test_bigram_batched_through_the_c_abi(bigram_model):
    """32 two-token prompts in one qd_prefill, then two qd_decode_step calls at B=32."""
    m, w, fed, dup = bigram_model
    B = 32
    prompts = [np.array([fed[b], fed[B + b]], np.int32) for b in range(B)]
    nxt, lg = m.prefill(prompts, logits=True)
    torch.cuda.synchronize()
    rounds = [(lg, nxt, [B + b for b in range(B)])]
    for k in ([b for b in range(B)], [2 * B + b for b in range(B)]):
        nxt, lg = m.decode_step(torch.tensor(fed[k], dtype=torch.int32, device="cuda"), logits=True)
        torch.cuda.synchronize()
        rounds.append((lg, nxt, k))
    for lg, nxt, ks in rounds:
        got = lg.cpu().numpy().astype(np.float64)
        ids = nxt.cpu().numpy()
        for b, k in enumerate(ks):
            np.testing.assert_array_equal(got[b], _bigram_logits(w, fed[k]), err_msg=f"row {b}")
            assert ids[b] == dup[k], (b, ids[b], dup[k])
    say("[gpu] exact bigram B=32: prefill rows + 2 decode steps bit-exact, planted ties resolved")
