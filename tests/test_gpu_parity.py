"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every input is seeded and synthetic (workloads): N(0, 0.02^2) weights, uniform prompt
ids, at the Qwen3 family's shapes ("Model-agnostic LLM inference", section "Supported
models").  Quantization ("The quantized load cache") must be bit-exact; logits and ids
must meet the bar in parity.py.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import Oracle, quantize_model, quantize_rows
from workloads import SHAPES, ModelShape, make_weights, make_prompt, make_prompts
from parity import say, check_step, logit_err, margin_of, bar_for, STRICT_TOL, safe_draw as _safe_margins

pytestmark = pytest.mark.gpu

TINY = SHAPES["tiny"]
WIDE = ModelShape(hidden=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=64,
                  intermediate=256, vocab=512)
# ragged tails everywhere: vocab not a multiple of any tile, 3 query heads per KV head
ODD = ModelShape(hidden=96, n_layers=3, n_heads=6, n_kv_heads=2, head_dim=32,
                 intermediate=160, vocab=1000)


def _model(shape, weights, **kw):
    import int8_weight_only_amd as qd
    return qd.Model(shape, weights, **kw)


@pytest.fixture(scope="module")
def tiny_setup():
    w = make_weights(TINY, seed=0, gains="uniform")
    qm = quantize_model(w)
    say("[gpu] loading tiny model")
    m = _model(TINY, w, max_batch=4, max_ctx=128, max_prefill_tokens=256)
    yield TINY, w, qm, m
    m.close()


@pytest.mark.parametrize("shape", [TINY, WIDE, ODD], ids=["tiny", "wide", "odd"])
def test_quantization_bit_exact(shape):
    w = make_weights(shape, seed=3)
    say(f"[gpu] quantization bit-exact {shape}")
    m = _model(shape, w, max_batch=1, max_ctx=64, max_prefill_tokens=64)
    try:
        q, s = m.export_quantized("embed")
        qr, sr = quantize_rows(w["embed"])
        np.testing.assert_array_equal(s, sr)
        np.testing.assert_array_equal(q, qr)
        for li in range(shape.n_layers):
            for t in ("q", "k", "v", "o", "gate", "up", "down"):
                q, s = m.export_quantized(t, li)
                qr, sr = quantize_rows(w["layers"][li][t])
                np.testing.assert_array_equal(s, sr, err_msg=f"{t}{li}")
                np.testing.assert_array_equal(q, qr, err_msg=f"{t}{li}")
    finally:
        m.close()


def _teacher_forced(m, shape, qm, prompt, n_steps, label, config, orc=None):
    """Prefill + n_steps decode steps fed the oracle's ids; check every step."""
    if orc is None:
        orc = Oracle(shape, qm, mode="bf16").generate(prompt, n_steps + 1)
    nxt, lg = m.prefill([prompt], logits=True)
    torch.cuda.synchronize()
    errs = [check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][0], orc["margin"][0],
                       config, f"{label} prefill")]
    for k in range(1, n_steps + 1):
        feed = torch.tensor([orc["ids"][k - 1]], dtype=torch.int32, device="cuda")
        nxt, lg = m.decode_step(feed, logits=True)
        torch.cuda.synchronize()
        errs.append(check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][k],
                               orc["margin"][k], config, f"{label} step {k}"))
    strict = sum(e <= STRICT_TOL for e in errs)
    say(f"[gpu] {label}: max logit err {max(errs):.3g} (bar {bar_for(config)[0]}), "
        f"{strict}/{len(errs)} steps within {STRICT_TOL}")
    return errs


def test_teacher_forced_tiny(tiny_setup):
    shape, w, qm, m = tiny_setup
    say("[gpu] teacher-forced tiny, 16-token prompt, 16 steps")
    _teacher_forced(m, shape, qm, make_prompt(shape.vocab, 16, 1000), 16, "tiny", "tiny")


@pytest.mark.parametrize("shape,config", [(WIDE, "wide"), (ODD, "odd")], ids=["wide", "odd"])
def test_teacher_forced_other_shapes(shape, config):
    w = make_weights(shape, seed=1, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(shape.vocab, 77, 1001)
    orc = Oracle(shape, qm, mode="bf16").generate(prompt, 13)
    say(f"[gpu] teacher-forced {shape}")
    m = _model(shape, w, max_batch=2, max_ctx=200, max_prefill_tokens=200)
    try:
        # a prompt longer than one attention chunk, with a ragged tail
        _teacher_forced(m, shape, qm, prompt, 12, config, config, orc)
    finally:
        m.close()


def test_generate_greedy_matches_oracle(tiny_setup):
    shape, w, qm, m = tiny_setup
    prompt = make_prompt(shape.vocab, 16, 1000)
    say("[gpu] generate_greedy tiny 16+16")
    res = m.generate_greedy([prompt], 16)
    orc = Oracle(shape, qm, mode="bf16").generate(prompt, 16)
    got = res.generated[0]
    # identical up to the first step whose oracle margin is not decisive
    gate = bar_for("tiny")[1]
    for k in range(16):
        if orc["margin"][k] <= gate:
            break
        assert got[k] == orc["ids"][k], f"step {k}"
    assert res.token_ids[0][:16] == list(prompt)
    assert res.steps == 15 and res.decode_us > 0 and res.prefill_us > 0


@pytest.mark.parametrize("shape,config,seed", [(TINY, "tiny", 0), (WIDE, "wide", 1),
                                               (ODD, "odd", 1)], ids=["tiny", "wide", "odd"])
def test_generate_greedy_other_shapes(shape, config, seed):
    """Graph-replayed generate (24 new tokens: three 8-step graphs) gives the oracle's ids
    wherever the oracle's margin decides them, at three shapes."""
    w = make_weights(shape, seed=seed, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(shape.vocab, 40, 1020)
    say(f"[gpu] generate {config}, 40+24")
    m = _model(shape, w, max_batch=1, max_ctx=128, max_prefill_tokens=64)
    try:
        a = m.generate_greedy([prompt], 24)
    finally:
        m.close()
    assert a.steps == 23
    orc = Oracle(shape, qm, mode="bf16").generate(prompt, 24)
    for k in range(24):
        if orc["margin"][k] <= bar_for(config)[1]:
            break
        assert a.generated[0, k] == orc["ids"][k], k


def test_generate_repeat_is_deterministic(tiny_setup):
    shape, w, qm, m = tiny_setup
    prompt = make_prompt(shape.vocab, 20, 1002)
    say("[gpu] generate twice, compare")
    a = m.generate_greedy([prompt], 24).generated
    b = m.generate_greedy([prompt], 24).generated
    np.testing.assert_array_equal(a, b)


def test_batched_ragged_generate_matches_single(tiny_setup):
    """Each sequence's output is independent of the batch it runs in."""
    shape, w, qm, m = tiny_setup
    prompts = [make_prompt(shape.vocab, n, 1010 + i) for i, n in enumerate((16, 5, 33))]
    say("[gpu] batched ragged B=3")
    batched = m.generate_greedy(prompts, 12).generated
    for i, p in enumerate(prompts):
        single = m.generate_greedy([p], 12).generated[0]
        orc = Oracle(shape, qm, mode="bf16").generate(p, 12)
        for k in range(12):
            if orc["margin"][k] <= bar_for("tiny")[1]:
                break
            assert batched[i, k] == orc["ids"][k] == single[k], (i, k)


@pytest.mark.parametrize("xstage", [1, 0], ids=["row-staged", "operand-loads"])
def test_batched_teacher_forced_logits(xstage):
    """B=9 (one 16-row MFMA tile) teacher-forced against the oracle per sequence, with the
    activations loaded row-contiguously and reordered in LDS (default) or loaded directly
    in the operand layout."""
    shape = TINY
    w = make_weights(shape, seed=2, gains="uniform")
    qm = quantize_model(w)
    B = 9
    prompts = make_prompts(shape.vocab, 12, B, seed0=2000)
    say(f"[gpu] batched teacher-forced B=9, skinny_xstage={xstage}")
    m = _model(shape, w, max_batch=B, max_ctx=64, max_prefill_tokens=B * 12)
    try:
        m.set_tuning(skinny_xstage=xstage)
        orcs = [Oracle(shape, qm, mode="bf16").generate(p, 6) for p in prompts]
        nxt, lg = m.prefill(list(prompts), logits=True)
        torch.cuda.synchronize()
        for b in range(B):
            check_step(lg[b].cpu().numpy(), nxt[b].item(), orcs[b]["logits"][0],
                       orcs[b]["margin"][0], "tiny-b", f"b{b} prefill")
        for k in range(1, 6):
            feed = torch.tensor([o["ids"][k - 1] for o in orcs], dtype=torch.int32, device="cuda")
            nxt, lg = m.decode_step(feed, logits=True)
            torch.cuda.synchronize()
            for b in range(B):
                check_step(lg[b].cpu().numpy(), nxt[b].item(), orcs[b]["logits"][k],
                           orcs[b]["margin"][k], "tiny-b", f"b{b} step {k}")
    finally:
        m.close()


# hidden 288 and intermediate 544 are not multiples of 128: the last 128-k block of a
# split is partial; down (544 -> 288) splits five ways, q|k|v and gate|up three ways
SPLITK = ModelShape(hidden=288, n_layers=2, n_heads=6, n_kv_heads=2, head_dim=32,
                    intermediate=544, vocab=1000)


@pytest.mark.parametrize("B,split", [(3, 3), (20, 1), (20, 3), (33, 2)],
                         ids=["b3-all", "b20-off", "b20-all", "b33-few"])
def test_batched_split_k_teacher_forced(B, split):
    """Batched decode projections with K split over work-groups (last arrival adds the
    partials in split order) against the oracle per sequence, and against no split."""
    shape = SPLITK
    w = make_weights(shape, seed=5, gains="uniform")
    qm = quantize_model(w)
    prompts = [make_prompt(shape.vocab, 6 + (b % 5), 4000 + b) for b in range(B)]
    say(f"[gpu] batched split-K teacher-forced B={B} skinny_split={split}")
    m = _model(shape, w, max_batch=B, max_ctx=32, max_prefill_tokens=B * 12)
    try:
        m.set_tuning(skinny_split=split)
        orcs = [Oracle(shape, qm, mode="bf16").generate(p, 4) for p in prompts]
        m.prefill(prompts)
        for k in range(1, 4):
            feed = torch.tensor([o["ids"][k - 1] for o in orcs], dtype=torch.int32, device="cuda")
            nxt, lg = m.decode_step(feed, logits=True)
            torch.cuda.synchronize()
            for b in range(B):
                check_step(lg[b].cpu().numpy(), nxt[b].item(), orcs[b]["logits"][k],
                           orcs[b]["margin"][k], "splitk", f"b{b} step {k}")
    finally:
        m.close()


@pytest.mark.parametrize("B,norm", [(20, 1), (20, 0), (12, 1)], ids=["b20-folded", "b20-separate", "b12-folded"])
def test_batched_folded_norm_teacher_forced(B, norm):
    """hidden 512: the RMSNorm before q|k|v and gate|up runs inside the batched projection
    (two 16-token tiles at B=20, one at B=12) or as its own launch; both against the oracle."""
    w = make_weights(MID, seed=6, gains="uniform")
    qm = quantize_model(w)
    prompts = [make_prompt(MID.vocab, 6 + (b % 4), 5000 + b) for b in range(B)]
    say(f"[gpu] batched folded-norm teacher-forced B={B} skinny_norm={norm}")
    m = _model(MID, w, max_batch=B, max_ctx=32, max_prefill_tokens=B * 12)
    try:
        m.set_tuning(skinny_norm=norm)
        orcs = [Oracle(MID, qm, mode="bf16").generate(p, 4) for p in prompts]
        m.prefill(prompts)
        for k in range(1, 4):
            feed = torch.tensor([o["ids"][k - 1] for o in orcs], dtype=torch.int32, device="cuda")
            nxt, lg = m.decode_step(feed, logits=True)
            torch.cuda.synchronize()
            for b in range(B):
                check_step(lg[b].cpu().numpy(), nxt[b].item(), orcs[b]["logits"][k],
                           orcs[b]["margin"][k], "mid", f"b{b} step {k}")
    finally:
        m.close()


def test_error_paths_do_no_gpu_work(tiny_setup):
    import int8_weight_only_amd as qd
    shape, w, qm, m = tiny_setup
    with pytest.raises(qd.QdError) as e:
        m.generate_greedy([np.array([], np.int32)], 4)
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        m.generate_greedy([np.array([shape.vocab], np.int32)], 4)
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        m.generate_greedy([np.array([1, 2], np.int32)], 0)
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        m.generate_greedy([np.array([1, 2], np.int32)], 200)  # past max_ctx 128
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        m.generate_greedy([np.array([1, 2], np.int32)] * 5, 4)  # past max_batch
    assert e.value.code == "invalid_arguments"
    bad = {"embed": w["embed"], "final_norm": w["final_norm"],
           "layers": [dict(L) for L in w["layers"]]}
    bad["layers"][1]["down"] = None
    with pytest.raises(qd.QdError) as e:
        qd.Model(shape, bad, max_batch=1, max_ctx=32, max_prefill_tokens=32)
    assert e.value.code == "checkpoint_not_found" and "layers.1.down_proj" in str(e.value)


def test_large_batch_teacher_forced_logits():
    """B=40 runs the skinny MFMA path with four 16-token tiles."""
    shape = TINY
    w = make_weights(shape, seed=2, gains="uniform")
    qm = quantize_model(w)
    B = 40
    prompts = [make_prompt(shape.vocab, 5 + (b % 7), 3000 + b) for b in range(B)]
    say("[gpu] batched teacher-forced B=40, ragged prompts")
    m = _model(shape, w, max_batch=B, max_ctx=32, max_prefill_tokens=B * 12)
    try:
        orcs = [Oracle(shape, qm, mode="bf16").generate(p, 3) for p in prompts]
        nxt, lg = m.prefill(prompts, logits=True)
        torch.cuda.synchronize()
        for k in range(3):
            if k:
                feed = torch.tensor([o["ids"][k - 1] for o in orcs], dtype=torch.int32, device="cuda")
                nxt, lg = m.decode_step(feed, logits=True)
                torch.cuda.synchronize()
            for b in range(B):
                check_step(lg[b].cpu().numpy(), nxt[b].item(), orcs[b]["logits"][k],
                           orcs[b]["margin"][k], "tiny-b", f"b{b} step {k}")
    finally:
        m.close()


MID = ModelShape(hidden=512, n_layers=2, n_heads=8, n_kv_heads=4, head_dim=128,
                 intermediate=1024, vocab=4096)


def test_teacher_forced_mid_split_k():
    """hidden 512 / head_dim 128: prefill GEMMs take the split-K path, flash prefill D=128."""
    w = make_weights(MID, seed=4, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(MID.vocab, 200, 1004)
    orc = Oracle(MID, qm, mode="bf16").generate(prompt, 8)
    say("[gpu] teacher-forced mid (split-K prefill), 200-token prompt")
    m = _model(MID, w, max_batch=2, max_ctx=256, max_prefill_tokens=512)
    try:
        _teacher_forced(m, MID, qm, prompt, 7, "mid", "mid", orc)
    finally:
        m.close()


@pytest.mark.parametrize("rows", [64, 128])
def test_prefill_attention_tile_rows(rows):
    """200-token prompt with prefill attention query tiles of 64 rows (4 tiles) or 128 rows
    (two row groups per wave; tiles of 128 and a ragged 72), against the oracle; later
    layers read every row's attention output through the K/V cache."""
    w = make_weights(MID, seed=4, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(MID.vocab, 200, 1004)
    orc = Oracle(MID, qm, mode="bf16").generate(prompt, 3)
    say(f"[gpu] mid prefill attention with {rows}-row tiles")
    m = _model(MID, w, max_batch=1, max_ctx=256, max_prefill_tokens=256)
    try:
        m.set_tuning(flash_rows=rows)
        _teacher_forced(m, MID, qm, prompt, 2, f"mid tiles{rows}", "mid", orc)
    finally:
        m.close()


@pytest.mark.parametrize("n_prompt", [64, 100])
def test_prefill_few_rows_both_gemm_kernels(n_prompt):
    """Prompts of one and two 64-row tiles (100: ragged): the prefill projections through the
    k-sliced kernel (default at <= 128 rows; O and down as 4 k-split partials at this
    shape) and through the k-stepped kernel (prefill_gemm=0), each against the oracle."""
    w = make_weights(MID, seed=4, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(MID.vocab, n_prompt, 1004)
    orc = Oracle(MID, qm, mode="bf16").generate(prompt, 1)
    m = _model(MID, w, max_batch=1, max_ctx=256, max_prefill_tokens=256)
    try:
        for mode, name in ((1, "k-sliced"), (0, "k-stepped")):
            say(f"[gpu] mid prefill, {n_prompt} rows, {name} GEMM")
            m.set_tuning(prefill_gemm=mode)
            nxt, lg = m.prefill([prompt], logits=True)
            torch.cuda.synchronize()
            check_step(lg[0].cpu().numpy(), nxt[0].item(), orc["logits"][0], orc["margin"][0],
                       "mid", f"mid {n_prompt} rows {name}")
    finally:
        m.close()


ROPE64 = ModelShape(hidden=256, n_layers=2, n_heads=16, n_kv_heads=8, head_dim=64,
                    intermediate=512, vocab=1000)


@pytest.mark.parametrize("mode", [1, 0], ids=["fused-rope", "separate-rope"])
def test_prefill_qkv_epilogue_rope_head_dim_64(mode):
    """2048-token prompt, head_dim 64, 32 q|k|v heads: the q|k|v projection runs as 256
    tiles of 128x128 (two heads each); mode 1 does the QK-norm, RoPE and K/V cache writes
    in that GEMM's epilogue, mode 0 in the separate launch.  Two teacher-forced decode steps
    read the K/V rows the prefill wrote."""
    w = make_weights(ROPE64, seed=6, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(ROPE64.vocab, 2048, 1006)
    orc = Oracle(ROPE64, qm, mode="bf16").generate(prompt, 3)
    say(f"[gpu] rope64 2048-token prefill, prefill_gemm={mode}")
    m = _model(ROPE64, w, max_batch=1, max_ctx=2064, max_prefill_tokens=2048)
    try:
        m.set_tuning(prefill_gemm=mode)
        _teacher_forced(m, ROPE64, qm, prompt, 2, "rope64", "rope64", orc)
    finally:
        m.close()


def test_teacher_forced_long_context():
    """1500-token prompt: 24 prefill tiles per head; decode attention over many position
    splits (~24, merged by the last split or by the merge launch), then at most 2 splits
    (12 chunks each: the multi-chunk loop)."""
    w = make_weights(WIDE, seed=5, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(WIDE.vocab, 1500, 1005)
    orc = Oracle(WIDE, qm, mode="bf16").generate(prompt, 24)
    say("[gpu] teacher-forced long context: 1500-token prompt, 23 decode steps")
    m = _model(WIDE, w, max_batch=1, max_ctx=2048, max_prefill_tokens=2048)
    try:
        _teacher_forced(m, WIDE, qm, prompt, 23, "wide-long", "wide-long", orc)
        # the separate merge launch instead of the in-kernel merge by the last split (the
        # default)
        m.set_tuning(attn_merge_last=0)
        _teacher_forced(m, WIDE, qm, prompt, 23, "wide-long merge launch", "wide-long", orc)
        m.set_tuning(attn_merge_last=1)
        m.set_tuning(attn_max_splits=2)
        _teacher_forced(m, WIDE, qm, prompt, 23, "wide-long 2 splits", "wide-long", orc)
    finally:
        m.close()


def test_decode_attention_merge_in_o_projection():
    """Single-row decode at 250..255 positions (four position splits): by default the O
    projection merges the attention's split partials as it loads its input; with merge
    mode 2 the attention's last split merges them.  Both follow the oracle, and since both
    merges add the splits in the same order with the same arithmetic, their logits are
    bit-identical."""
    w = make_weights(MID, seed=7, gains="uniform")
    qm = quantize_model(w)
    prompt = make_prompt(MID.vocab, 250, 1007)
    orc = Oracle(MID, qm, mode="bf16").generate(prompt, 6)
    say("[gpu] decode attention merged in the O projection vs by the last split")
    m = _model(MID, w, max_batch=1, max_ctx=320, max_prefill_tokens=320)
    try:
        runs = {}
        for mode in (1, 2):
            m.set_tuning(attn_merge_last=mode)
            _teacher_forced(m, MID, qm, prompt, 5, f"mid merge mode {mode}", "mid", orc)
            nxt, lg = m.prefill([prompt], logits=True)
            steps = [lg[0].cpu().numpy()]
            for k in range(1, 6):
                feed = torch.tensor([orc["ids"][k - 1]], dtype=torch.int32, device="cuda")
                nxt, lg = m.decode_step(feed, logits=True)
                steps.append(lg[0].cpu().numpy())
            torch.cuda.synchronize()
            runs[mode] = steps
        for k in range(6):
            np.testing.assert_array_equal(runs[1][k], runs[2][k], err_msg=f"step {k}")
    finally:
        m.set_tuning(attn_merge_last=1)
        m.close()


def test_continuous_batching_slots_teacher_forced():
    """Sequences join and leave a running batch ("LLM inference overview", section
    "Results": continuous batching): prompts are prefilled into free KV slots while other
    slots are mid-decode, and each decode step lists its slots in any order, each at its
    own length.  Every sequence's logits follow the oracle run of that sequence alone."""
    import int8_weight_only_amd as qd
    shape = TINY
    w = make_weights(shape, seed=7, gains="uniform")
    qm = quantize_model(w)
    lens = {"A": 7, "B": 12, "C": 5, "D": 9}
    prompts = {s: make_prompt(shape.vocab, n, 6000 + i) for i, (s, n) in enumerate(lens.items())}
    need = {"A": 6, "B": 7, "C": 7, "D": 4}
    orcs = {s: Oracle(shape, qm, mode="bf16").generate(prompts[s], need[s]) for s in prompts}
    step = {s: 0 for s in prompts}
    say("[gpu] continuous batching through slot-addressed prefill and decode")
    m = _model(shape, w, max_batch=5, max_ctx=64, max_prefill_tokens=64)

    def check(seq, lg_row, nxt_id):
        k = step[seq]
        check_step(lg_row, nxt_id, orcs[seq]["logits"][k], orcs[seq]["margin"][k], "tiny",
                   f"{seq} step {k}")
        step[seq] += 1

    def prefill(pairs):  # [(seq, slot)]
        nxt, lg = m.prefill([prompts[s] for s, _ in pairs], logits=True,
                            slots=[sl for _, sl in pairs])
        torch.cuda.synchronize()
        for i, (s, _) in enumerate(pairs):
            check(s, lg[i].cpu().numpy(), nxt[i].item())

    def decode(pairs):  # [(seq, slot)], rows in this order
        feed = torch.tensor([orcs[s]["ids"][step[s] - 1] for s, _ in pairs], dtype=torch.int32,
                            device="cuda")
        nxt, lg = m.decode_step(feed, logits=True, slots=[sl for _, sl in pairs])
        torch.cuda.synchronize()
        for i, (s, _) in enumerate(pairs):
            check(s, lg[i].cpu().numpy(), nxt[i].item())

    try:
        prefill([("A", 2)])
        decode([("A", 2)])
        decode([("A", 2)])
        prefill([("B", 0), ("C", 4)])           # two joins in one ragged prefill
        for _ in range(3):
            decode([("C", 4), ("A", 2), ("B", 0)])  # rows in slot-shuffled order
        prefill([("D", 2)])                      # A leaves, D takes its slot
        for _ in range(2):
            decode([("B", 0), ("D", 2), ("C", 4)])
        decode([("D", 2)])                       # the others idle this step
        decode([("C", 4), ("B", 0)])
        assert step == need, step
        # error paths: checked on the host before any GPU work
        feed = torch.zeros(2, dtype=torch.int32, device="cuda")
        for bad in ([0, 0], [0, 5], [0, 1]):     # duplicate, out of range, empty slot
            with pytest.raises(qd.QdError) as e:
                m.decode_step(feed, slots=bad)
            assert e.value.code == "invalid_arguments", bad
        with pytest.raises(qd.QdError) as e:
            m.prefill([prompts["A"], prompts["C"]], slots=[3, 3])
        assert e.value.code == "invalid_arguments"
        assert step == need  # the refused calls changed nothing on the host side
    finally:
        m.close()


SAMPLING = dict(temperature=0.8, top_k=40, min_p=0.05, top_p=0.9, repeat_penalty=1.3,
                presence_penalty=0.2, frequency_penalty=0.1)


# the second set keeps nearly the whole vocabulary: too many candidates lie far from the
# largest logit, so the device sampler takes its whole-row select path
SAMPLING_WIDE = dict(temperature=1.5, top_k=1000, min_p=0.0, top_p=0.95, repeat_penalty=1.1,
                     presence_penalty=0.0, frequency_penalty=0.05)


@pytest.mark.parametrize("params", [SAMPLING, SAMPLING_WIDE], ids=["top40", "top1000"])
def test_device_sampler_matches_oracle_on_its_own_logits(params):
    """The sampling chain ("Model-agnostic LLM inference", section "Sampling") on the
    device against the oracle's, both fed the GPU's fp32 logits, the token counts of
    each sequence and the Philox draw for its seed: the drawn ids must agree wherever no
    decision sits within 1e-5 of a boundary (fp32 against fp64)."""
    from oracle.sampling import SamplingParams, draw_uniform
    shape = TINY
    w = make_weights(shape, seed=8, gains="uniform")
    B = 3
    prompts = [make_prompt(shape.vocab, 9 + 3 * b, 7000 + b) for b in range(B)]
    seeds = [11, 2 ** 63 + 5, 33]
    p = SamplingParams(**params)
    say(f"[gpu] device sampler vs oracle sampler, top_k {params['top_k']}")
    m = _model(shape, w, max_batch=B, max_ctx=64, max_prefill_tokens=64)
    try:
        counts = [np.bincount(pr, minlength=shape.vocab) for pr in prompts]
        _, lg = m.prefill(prompts, logits=True)
        checked = total = 0
        for step in range(10):
            ids = m.sample(lg, seeds, **params)
            torch.cuda.synchronize()
            got = ids.cpu().numpy()
            rows = lg.cpu().numpy().astype(np.float64)
            for b in range(B):
                want, safe = _safe_margins(rows[b], counts[b], p, draw_uniform(seeds[b], step))
                total += 1
                if safe:
                    checked += 1
                    assert got[b] == want, f"row {b} step {step}: device {got[b]} oracle {want}"
                counts[b][got[b]] += 1
            _, lg = m.decode_step(ids, logits=True)
        say(f"[gpu] sampler: {checked}/{total} draws clear of every boundary, all equal")
        assert checked >= 0.8 * total
    finally:
        m.close()


def test_top_k_one_sampling_is_the_greedy_sequence(tiny_setup):
    """top_k = 1 at any temperature reproduces the greedy sequence exactly (the pages'
    stated property of the sampling chain)."""
    shape, w, qm, m = tiny_setup
    prompt = make_prompt(shape.vocab, 11, 7100)
    greedy = m.generate_greedy([prompt], 10).generated[0]
    for T in (0.3, 2.0):
        _, lg = m.prefill([prompt], logits=True)
        got = []
        for _ in range(10):
            ids = m.sample(lg, [1234], temperature=T, top_k=1)
            got.append(int(ids[0].item()))
            _, lg = m.decode_step(ids, logits=True)
        assert got == [int(x) for x in greedy], (T, got, greedy)


def test_sampling_repeats_with_the_seed_in_any_slot():
    """Same prompt, parameters and seed give the same tokens, whichever KV slot the
    sequence occupies; another seed gives another sequence."""
    shape = TINY
    w = make_weights(shape, seed=9, gains="uniform")
    prompt = make_prompt(shape.vocab, 10, 7200)
    m = _model(shape, w, max_batch=4, max_ctx=64, max_prefill_tokens=64)

    def run(slot, seed):
        _, lg = m.prefill([prompt], logits=True, slots=[slot])
        out = []
        for _ in range(12):
            ids = m.sample(lg, [seed], slots=[slot], temperature=1.5, top_k=200, top_p=0.98)
            out.append(int(ids[0].item()))
            _, lg = m.decode_step(ids, logits=True, slots=[slot])
        return out

    try:
        a, b, c = run(0, 77), run(3, 77), run(1, 78)
        assert a == b
        assert a != c
    finally:
        m.close()


def test_sampler_rejects_bad_parameters(tiny_setup):
    import int8_weight_only_amd as qd
    shape, w, qm, m = tiny_setup
    _, lg = m.prefill([make_prompt(shape.vocab, 5, 7300)], logits=True)
    for bad in (dict(temperature=0.0), dict(top_k=0), dict(top_k=1025), dict(min_p=1.5),
                dict(top_p=0.0), dict(repeat_penalty=0.0)):
        with pytest.raises(qd.QdError) as e:
            m.sample(lg, [1], **bad)
        assert e.value.code == "invalid_arguments", bad


def test_quantized_load_cache_round_trip(tmp_path):
    """The quantized load cache ("Model-agnostic LLM inference", section "The quantized
    load cache"): a model restored from the cache holds bit-identical codes and scales and
    generates the identical greedy sequence; another checkpoint's digest or a damaged
    file is refused with cache_miss."""
    import hashlib
    import int8_weight_only_amd as qd
    shape = ODD
    w = make_weights(shape, seed=10, gains="uniform")
    digest = hashlib.sha256(b"odd checkpoint, seed 10").digest()
    path = str(tmp_path / "weights_i8.cache")
    say("[gpu] quantized load cache round trip")
    a = _model(shape, w, max_batch=2, max_ctx=64, max_prefill_tokens=64)
    try:
        a.save_cache(path, digest)
        b = _model(shape, None, max_batch=2, max_ctx=64, max_prefill_tokens=64,
                   cache_path=path, source_digest=digest)
        try:
            for t in ("embed",) + tuple((n, l) for l in range(shape.n_layers)
                                        for n in ("q", "k", "v", "o", "gate", "up", "down")):
                name, layer = (t, 0) if isinstance(t, str) else t
                qa, sa = a.export_quantized(name, layer)
                qb, sb = b.export_quantized(name, layer)
                np.testing.assert_array_equal(qa, qb)
                np.testing.assert_array_equal(sa, sb)
            prompt = make_prompt(shape.vocab, 13, 7400)
            ga = a.generate_greedy([prompt], 12).generated
            gb = b.generate_greedy([prompt], 12).generated
            np.testing.assert_array_equal(ga, gb)
        finally:
            b.close()
        with pytest.raises(qd.QdError) as e:
            _model(shape, None, max_batch=2, max_ctx=64, max_prefill_tokens=64, cache_path=path,
                   source_digest=hashlib.sha256(b"another checkpoint").digest())
        assert e.value.code == "cache_miss"
        raw = bytearray(open(path, "rb").read())
        raw[-1] ^= 0xFF
        open(path, "wb").write(bytes(raw))
        with pytest.raises(qd.QdError) as e:
            _model(shape, None, max_batch=2, max_ctx=64, max_prefill_tokens=64, cache_path=path,
                   source_digest=digest)
        assert e.value.code == "cache_miss" and "SHA-256" in str(e.value)
    finally:
        a.close()
