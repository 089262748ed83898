"""GPU parity against the oracle at the Qwen3-0.6B shape (every width, head count and the
151,936-token vocabulary; 2 layers so the oracle finishes in seconds).

The kernels a decode step launches, their tile shapes and work splits depend on the
widths, heads, vocabulary, batch and context, not on the number of layers, so these runs
take the same code paths as the 28-layer model ("Run local LLM decode", section
"Limitations": the Qwen3-0.6B-Base dimensions):
  * B = 1: the register GEMV for q|k|v, O, gate/up and down, the LM head's grid-capped
    row-block loop over 151,936 rows with its fused arg-max, decode attention in 5 splits;
  * B = 8, 16 and 32: the MFMA skinny projections (RMSNorm folded into q|k|v and gate/up;
    at 32 rows the O and down projections split over K across work-groups), the batched LM
    head, and at B = 32 (32 x 8 KV heads = 256 pairs) the eight-wave attention kernel; their
    prompts prefilled together (M = 2048, 4096, 8192) take the three many-row GEMMs;
  * an 8192-token prompt: flash prefill over 128 query tiles per head, then decode
    attention over about 43 position splits (split count from the measured residency) merged by the last split (and, in a second run, by
    the separate merge launch).
Every step is teacher-forced on the oracle's ids; logits meet the bar in parity.py and
each test prints its error against the strict 2e-2 beside the bar.  Synthetic inputs
(workloads): N(0, 0.02^2) weights, gains from U(0.5, 1.5), uniform prompt ids.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import Oracle, quantize_model
from workloads import SHAPES, make_weights, make_prompt
from parity import say, check_step, bar_for, STRICT_TOL, logit_err

pytestmark = pytest.mark.gpu

SH = dataclasses.replace(SHAPES["qwen3-0.6b"], n_layers=2)
LONG = 8192


@pytest.fixture(scope="module")
def full_setup():
    import int8_weight_only_amd as qd
    say("[gpu] fullsize: drawing Qwen3-0.6B-shape weights (2 layers)")
    w = make_weights(SH, seed=0, gains="uniform")
    qm = quantize_model(w)
    say("[gpu] fullsize: loading the model (max_batch 32, max_ctx 8200)")
    m = qd.Model(SH, w, max_batch=32, max_ctx=LONG + 8, max_prefill_tokens=LONG)
    yield w, qm, m
    m.close()


def _report(label, errs, config):
    strict = sum(e <= STRICT_TOL for e in errs)
    say(f"[gpu] {label}: max logit err {max(errs):.4g} (bar {bar_for(config)[0]}, strict "
        f"{STRICT_TOL}: {strict}/{len(errs)} steps within)")


def test_fullsize_embedding_rows_bit_exact(full_setup):
    """The embedding is one multiply and one rounding: bf16(code x row scale), bit-exact."""
    w, qm, m = full_setup
    ids = np.array([0, 1, 77777, 151935, 4242, 100000, 31, 150000], np.int32)
    got = m.run_op("embed", torch.as_tensor(ids).cuda()).float().cpu().numpy()
    want = Oracle(SH, qm).embed(ids)
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_fullsize_b1_teacher_forced(full_setup):
    w, qm, m = full_setup
    prompt = make_prompt(SH.vocab, 256, 1000)
    say("[gpu] fullsize B=1: oracle, 256-token prompt + 4 steps")
    orc = Oracle(SH, qm).generate(prompt, 5)
    nxt, lg = m.prefill([prompt], logits=True)
    torch.cuda.synchronize()
    errs = [check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][0], orc["margin"][0],
                       "qwen3-0.6b-l2", "B=1 prefill")]
    for k in range(1, 5):
        feed = torch.tensor([orc["ids"][k - 1]], dtype=torch.int32, device="cuda")
        nxt, lg = m.decode_step(feed, logits=True)
        torch.cuda.synchronize()
        errs.append(check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][k],
                               orc["margin"][k], "qwen3-0.6b-l2", f"B=1 step {k}"))
    _report("fullsize B=1 (prefill row + 4 steps)", errs, "qwen3-0.6b-l2")


@pytest.mark.parametrize("B", [8, 16, 32])
def test_fullsize_batched_teacher_forced(full_setup, B):
    """B prompts of 256 tokens prefilled together (M = 256 B), then 3 decode steps; rows 0,
    B/2 and B-1 are teacher-forced against their own oracle runs, every row's fused arg-max
    is checked against the arg-max of its own logits.  The prefill GEMMs: M = 2048 runs the
    128x128-tile kernel for q|k|v (QK-norm/RoPE epilogue) and gate/up; M = 4096 the direct-
    load kernel for those and the 128x128 kernel's residual epilogue for O and down; M = 8192
    the direct-load kernel for every projection."""
    w, qm, m = full_setup
    prompts = [make_prompt(SH.vocab, 256, 1000 + b) for b in range(B)]
    rows = [0, B // 2, B - 1]
    say(f"[gpu] fullsize B={B}: oracle for rows {rows}")
    orcs = {b: Oracle(SH, qm).generate(prompts[b], 4) for b in rows}
    nxt, lg = m.prefill(prompts, logits=True)
    torch.cuda.synchronize()
    errs = []
    for k in range(4):
        if k:
            feed = nxt.clone()
            for b in rows:
                feed[b] = int(orcs[b]["ids"][k - 1])
            nxt, lg = m.decode_step(feed, logits=True)
            torch.cuda.synchronize()
        lgc = lg.cpu().numpy()
        ids = nxt.cpu().numpy()
        assert np.array_equal(ids, np.argmax(lgc, axis=1)), f"B={B} step {k}: fused arg-max"
        for b in rows:
            errs.append(check_step(lgc[b], ids[b], orcs[b]["logits"][k], orcs[b]["margin"][k],
                                   "qwen3-0.6b-l2", f"B={B} row {b} step {k}"))
    _report(f"fullsize B={B} (rows {rows}, prefill row + 3 steps)", errs, "qwen3-0.6b-l2")


def test_fullsize_long_context_merge_modes(full_setup):
    """8192-token prompt, 3 decode steps at 8193..8195 positions: 43 attention splits of
    192 positions, merged by the last split to finish (default) and by the merge launch."""
    w, qm, m = full_setup
    prompt = make_prompt(SH.vocab, LONG, 1005)
    say("[gpu] fullsize long context: oracle, 8192-token prompt + 3 steps")
    orc = Oracle(SH, qm).generate(prompt, 4)
    try:
        for merge_last in (1, 0):
            m.set_tuning(attn_merge_last=merge_last)
            nxt, lg = m.prefill([prompt], logits=True)
            torch.cuda.synchronize()
            errs = [check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][0],
                               orc["margin"][0], "long-0.6b-l2", "long prefill")]
            for k in range(1, 4):
                feed = torch.tensor([orc["ids"][k - 1]], dtype=torch.int32, device="cuda")
                nxt, lg = m.decode_step(feed, logits=True)
                torch.cuda.synchronize()
                errs.append(check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][k],
                                       orc["margin"][k], "long-0.6b-l2",
                                       f"long step {k} merge_last={merge_last}"))
            _report(f"fullsize long context, merge_last={merge_last}", errs, "long-0.6b-l2")
    finally:
        m.set_tuning(attn_merge_last=1)
