"""Benchmark of the int8 weight-only Qwen3-0.6B-shape forward step on one MI355X.

One step = one qd_generate_greedy call: prefill of a 256-token prompt, then 127 greedy
decode steps (128 generated tokens) at B=1, inputs resident in HBM.  Before timing,
a sampled full-size parity check against the CPU oracle must pass (bit-exact int8
codes and scales on sampled matrices; teacher-forced logits of the prefill row and the
first decode steps within the bar of tests/golden/noise_floor.json).  The oracle run
doubles as the CPU baseline.  Prints one JSON line.

Workloads come from "LLM inference overview" (sections "Results" and "Workload
characteristics"): prefill of a 256-token prompt, single-stream decode, batched decode
at B = 8..32 sweeping the weights once per step.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B] [--no-extra]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes_per_step(s, B, ctx):
    """Algorithmic HBM bytes of one decode step at batch B with ctx positions attended:
    every int8 weight, fp32 scale and fp32 gain once, plus K/V reads and writes."""
    d, H, KV, D, I, V, L = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab, s.n_layers
    rows_cols = [(H * D + 2 * KV * D, d), (d, H * D), (2 * I, d), (d, I)]
    w = L * (sum(r * c + 4 * r for r, c in rows_cols) + 4 * (2 * d + 2 * D)) + V * d + 4 * V + 4 * d
    kv = B * L * KV * D * 2 * 2 * ctx + B * L * KV * D * 2 * 2
    return w + kv


def kernel_bytes(s, B, ctx):
    """Algorithmic bytes per launch of each decode kernel class (weights + activations)."""
    d, H, KV, D, I, V = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab
    nqkv = H * D + 2 * KV * D
    return {
        "qkv": nqkv * d + 4 * nqkv + 4 * d + B * (2 * d + 2 * nqkv),
        "o": d * H * D + 4 * d + B * (2 * H * D + 4 * d),
        "gateup": 2 * I * d + 8 * I + 4 * d + B * (2 * d + 2 * I),
        "down": d * I + 4 * d + B * (2 * I + 4 * d),
        "lmhead": V * d + 4 * V + 4 * d + B * 2 * d,
        "attn": B * (KV * D * 2 * 2 * ctx + 4 * H * D),
        "rope": B * (4 * nqkv + 2 * 2 * KV * D),
        "embed": B * (d + 4 + 2 * d),
    }


def prefill_flops(s, M):
    d, H, KV, D, I, V, L = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab, s.n_layers
    gemm = 2 * M * d * (H * D + 2 * KV * D) + 2 * M * H * D * d + 2 * M * d * 2 * I + 2 * M * I * d
    attn = 4 * H * D * (M * (M + 1) // 2)
    return L * (gemm + attn) + 2 * d * V


KERNEL_SOURCES = [os.path.join(ROOT, "int8_weight_only_amd", "csrc", f)
                  for f in ("qd_common.h", "qd_device.h", "qd_kernels.hip", "qd_sample.hip")]


def kernel_source_sha() -> str:
    """sha256 over the device sources, in a fixed order (a traffic summary is valid only for
    the sources it was measured on)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(path, kernel_class):
    """HBM bytes per launch of a decode kernel class from a committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or None when the
    summary is missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"kernel source sha256: {kernel_source_sha()}" not in text:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == kernel_class:
            try:
                return int(cells[3])
            except ValueError:
                return None
    return None


def cpu_info():
    """CPU model name and the BLAS threads numpy uses (threadpoolctl), for cpu_baseline."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 0) for i in threadpool_info()
                    if i.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    return model, blas


def check_quantization(model, shape, w, layers):
    """Quantized codes and scales of the embedding and every matrix of ``layers`` against
    the oracle's quantizer, bit-exact."""
    from oracle import quantize_rows
    t = time.time()
    samples = [("embed", 0)] + [(m, l) for l in layers
                                for m in ("q", "k", "v", "o", "gate", "up", "down")]
    for name, layer in samples:
        q, s = model.export_quantized(name, layer)
        src = w["embed"] if name == "embed" else w["layers"][layer][name]
        qr, sr = quantize_rows(src)
        if not (np.array_equal(q, qr) and np.array_equal(s, sr)):
            raise SystemExit(f"parity gate failed: quantized {name}[{layer}] differs")
    log(f"[bench] quantization bit-exact on {len(samples)} matrices ({time.time() - t:.1f}s)")
    return len(samples)


class OracleRuns:
    """Greedy oracle runs of one model, one per prompt: logits and top-1/top-2 margins of
    the prefill row and of each decode step fed the oracle's own previous id.  Runs are
    extended on demand and timed (the decode steps double as the CPU baseline)."""

    def __init__(self, shape, w):
        from oracle import Oracle, quantize_model
        t = time.time()
        self.orc = Oracle(shape, quantize_model(w), mode="bf16")
        self.runs = {}
        self.t_pre = self.t_dec = 0.0
        self.n_pre = self.n_dec = 0
        log(f"[bench] oracle ready in {time.time() - t:.1f}s")

    def get(self, key, prompt, n):
        """(ids, logits, margins) of the first n generated positions of ``prompt``."""
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import margin_of
        r = self.runs.get(key)
        if r is None:
            seq = self.orc.new_sequence()
            t = time.time()
            lg = self.orc.forward(seq, prompt)
            self.t_pre += time.time() - t
            self.n_pre += len(prompt)
            r = {"seq": seq, "ids": [int(np.argmax(lg))], "logits": [lg], "margin": [margin_of(lg)]}
            self.runs[key] = r
        while len(r["ids"]) < n:
            t = time.time()
            lg = self.orc.forward(r["seq"], [r["ids"][-1]])
            self.t_dec += time.time() - t
            self.n_dec += 1
            r["ids"].append(int(np.argmax(lg)))
            r["logits"].append(lg)
            r["margin"].append(margin_of(lg))
        return r["ids"][:n], r["logits"][:n], r["margin"][:n]


def rows_gate(model, runs, prompts, keys, rows, n_steps, config, slots=None):
    """Teacher-forced parity of a batched prefill and n_steps decode steps: rows ``rows``
    are fed their oracle's ids and compared with it (logits within the bar of ``config``,
    ids equal where the oracle's margin passes the gate); every row's fused arg-max must
    equal the arg-max of its own logits.  slots: KV slot of each prompt (slot-addressed
    calls, rows shuffled on every decode step)."""
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import logit_err, bar_for, STRICT_TOL
    bar, gate = bar_for(config)
    orcs = {b: runs.get(keys[b], prompts[b], n_steps + 1) for b in rows}
    nxt, lg = model.prefill(list(prompts), logits=True, slots=slots)
    errs, exact, ids_ok = [], True, True
    rng = np.random.default_rng(5)
    order = np.arange(len(prompts))
    for k in range(n_steps + 1):
        if k:
            feed = nxt.clone()
            for b in rows:
                feed[int(np.where(order == b)[0][0])] = orcs[b][0][k - 1]
            if slots is not None:
                perm = rng.permutation(len(prompts))
                pidx = torch.as_tensor(perm, device="cuda").long()
                nxt, lg = model.decode_step(feed[pidx], logits=True,
                                            slots=[slots[order[i]] for i in perm])
                order = order[perm]
            else:
                nxt, lg = model.decode_step(feed, logits=True)
        lgc = lg.cpu().numpy()
        ids = nxt.cpu().numpy()
        exact &= bool(np.array_equal(ids, np.argmax(lgc, axis=1)))
        for b in rows:
            i = int(np.where(order == b)[0][0])
            errs.append(logit_err(lgc[i], orcs[b][1][k]))
            if orcs[b][2][k] > gate:
                ids_ok &= int(ids[i]) == orcs[b][0][k]
    rec = {"checked": "oracle", "rows": list(rows), "steps": n_steps + 1,
           "max_logit_err": round(max(errs), 5), "bar": bar,
           "within_strict_2e-2": f"{sum(e <= STRICT_TOL for e in errs)}/{len(errs)}",
           "fused_argmax_exact": exact, "ids_match_where_margin": ids_ok}
    if max(errs) > bar or not exact or not ids_ok:
        raise SystemExit(f"parity gate failed ({config}): {rec}")
    return rec


def free_run_gate(runs, key, prompt, gpu_ids, config, max_steps=32):
    """Free-running check: the GPU's greedy ids of one sequence equal the oracle's greedy
    ids up to the oracle's first low-margin step (there, either id is a valid arg-max
    within the bar); returns the number of leading steps checked."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import bar_for
    gate = bar_for(config)[1]
    n = min(max_steps, len(gpu_ids))
    ids, _, margins = runs.get(key, prompt, n)
    upto = next((k for k in range(n) if margins[k] <= gate), n)
    if list(gpu_ids[:upto]) != ids[:upto]:
        first = next(k for k in range(upto) if gpu_ids[k] != ids[k])
        raise SystemExit(f"parity gate failed: free-running ids differ from the oracle at step "
                         f"{first} (margin {margins[first]:.3g} > gate {gate})")
    return upto


def sampled_gate(model, shape, B, NP, seeds, params):
    """The first draw of a sampled run against the sampling oracle on the GPU's own fp32
    logits and token counts (the prompt's), at each row whose decision is clear of every
    boundary by 1e-5."""
    import torch
    from workloads import make_prompts
    from oracle.sampling import SamplingParams, draw_uniform
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import safe_draw
    prompts = make_prompts(shape.vocab, NP, B, seed0=1000)
    _, lg = model.prefill(list(prompts), logits=True)
    ids = model.sample(lg, seeds, **params).cpu().numpy()
    rows = lg.cpu().numpy().astype(np.float64)
    p = SamplingParams(**params)
    checked = 0
    for b in range(B):
        want, safe = safe_draw(rows[b], np.bincount(prompts[b], minlength=shape.vocab), p,
                               draw_uniform(seeds[b], 0))
        if safe:
            checked += 1
            if int(ids[b]) != int(want):
                raise SystemExit(f"parity gate failed: sampled row {b}: {ids[b]} != oracle {want}")
    return {"checked": "sampling oracle on the GPU's logits", "rows": B,
            "rows_clear_of_boundaries_equal": checked}


def consistency_gate(model, prompt, bar):
    """Full-size check where the oracle cannot run: the last row's logits from one prefill
    of the whole prompt against a prefill of all but the last token followed by one decode
    step of it (flash prefill attention vs split decode attention)."""
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import logit_err
    _, la = model.prefill([prompt], logits=True)
    model.prefill([prompt[:-1]])
    nb, lb = model.decode_step(torch.tensor([int(prompt[-1])], dtype=torch.int32,
                                            device="cuda"), logits=True)
    e = logit_err(lb[0].cpu().numpy(), la[0].cpu().numpy())
    ok = int(nb[0].item()) == int(np.argmax(lb[0].cpu().numpy()))
    parity = {"checked": "prefill-vs-decode", "max_logit_err": round(e, 5), "bar": bar,
              "fused_argmax_exact": bool(ok)}
    if e > bar or not ok:
        raise SystemExit(f"consistency gate failed: {parity}")
    return parity


def time_generate(model, prompts, new, steps, warmup):
    import torch
    for _ in range(warmup):
        model.generate_greedy(list(prompts), new)
    torch.cuda.synchronize()
    dev, pre, dec, res = [], [], [], None
    t0 = time.perf_counter()
    for _ in range(steps):
        res = model.generate_greedy(list(prompts), new)
        dev.append(res.prefill_us + res.decode_us)
        pre.append(res.prefill_us)
        dec.append(res.decode_us)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return float(np.mean(dev)), float(np.mean(pre)), float(np.mean(dec)), wall / steps, res


def time_cache_load(model, shape, max_batch, ctx, NP, load_s):
    """The quantized load cache ("Model-agnostic LLM inference", section "The quantized
    load cache"): wall time of a model load from fp32 host arrays (upload + quantize on
    the GPU) against a restore from the cache file (read + gate + upload), and the file
    size; the restored model's codes are compared with the loaded one's on two matrices."""
    import hashlib
    import tempfile
    import torch
    import int8_weight_only_amd as qd
    digest = hashlib.sha256(b"bench weights: seed 0, N(0, 0.02^2)").digest()
    d = tempfile.mkdtemp(prefix="qd_cache_")
    path = os.path.join(d, "weights_i8.cache")
    try:
        model.save_cache(path, digest)
        size = os.path.getsize(path)
        t = time.time()
        m2 = qd.Model(shape, None, max_batch=max_batch, max_ctx=ctx,
                      max_prefill_tokens=max_batch * NP, cache_path=path, source_digest=digest)
        torch.cuda.synchronize()
        cache_s = time.time() - t
        try:
            for name, layer in (("embed", 0), ("down", shape.n_layers - 1)):
                qa, sa = model.export_quantized(name, layer)
                qb, sb = m2.export_quantized(name, layer)
                assert np.array_equal(qa, qb) and np.array_equal(sa, sb), name
        finally:
            m2.close()
    finally:
        if os.path.exists(path):
            os.remove(path)
        os.rmdir(d)
    log(f"[bench] load: fp32 + quantize {load_s:.2f}s, cache {cache_s:.2f}s ({size / 1e9:.3f} GB)")
    return {"load_fp32_quantize_s": round(load_s, 3), "load_cache_s": round(cache_s, 3),
            "cache_bytes": size}


SAMPLED = dict(temperature=0.8, top_k=40, top_p=0.95, min_p=0.0, repeat_penalty=1.1)


def time_sampled(model, shape, B, NP, NN):
    """Sampled decode ("Model-agnostic LLM inference", section "Sampling", with the
    parameters of its example): B sequences, each step materializes the fp32 logits and
    draws every token through the device sampler (penalties, temperature, top-k, min-p,
    top-p, Philox draw).  Device time of the decode steps plus their draws."""
    import torch
    from workloads import make_prompts
    prompts = make_prompts(shape.vocab, NP, B, seed0=1000)
    seeds = [1234 + b for b in range(B)]
    steps = min(64, NN - 1)
    _, lg = model.prefill(list(prompts), logits=True)
    ids = model.sample(lg, seeds, **SAMPLED)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        _, lg = model.decode_step(ids, logits=True)
        ids = model.sample(lg, seeds, **SAMPLED)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    log(f"[bench] sampled B={B}: {steps} steps in {ms:.2f} ms")
    return {f"sampled_b{B}_tok_s": round(B * steps / (ms * 1e-3), 1)}


def time_continuous(model, shape, S, NP, NN):
    """Continuous batching ("LLM inference overview", section "Results"): S KV slots hold
    sequences of ragged lengths; every step lists all slots in a fresh random order
    (qd_decode_step_slots), and every 16 steps one sequence leaves and a new prompt is
    prefilled into its slot (qd_prefill_slots).  Device time of the whole schedule."""
    import torch
    from workloads import make_prompt
    rng = np.random.default_rng(7)
    lens = [NP // 2 + (NP // 2 - 4) * b // max(1, S - 1) for b in range(S)]
    steps = min(64, NN // 2)
    prompts = [make_prompt(shape.vocab, n, 3000 + b) for b, n in enumerate(lens)]
    order = rng.permutation(S)
    nxt, _ = model.prefill([prompts[i] for i in order], slots=order)
    ids = torch.empty(S, dtype=torch.int32, device="cuda")
    ids[torch.as_tensor(order, device="cuda").long()] = nxt  # ids indexed by slot
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    joins, dec_tok = 0, 0
    ev0.record()
    for k in range(steps):
        if k and k % 16 == 0:  # slot k % S leaves; a new prompt takes it
            sl = k % S
            jn, _ = model.prefill([make_prompt(shape.vocab, NP // 2, 3500 + k)], slots=[sl])
            ids[sl] = jn[0]
            joins += 1
        perm = rng.permutation(S)
        pidx = torch.as_tensor(perm, device="cuda").long()
        out, _ = model.decode_step(ids[pidx], slots=perm)
        ids[pidx] = out
        dec_tok += S
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    log(f"[bench] continuous S={S}: {dec_tok} decode tokens + {joins} joins in {ms:.2f} ms")
    return {f"continuous_s{S}_tok_s": round(dec_tok / (ms * 1e-3), 1),
            f"continuous_s{S}_schedule": f"{S} slots, prompts {lens[0]}..{lens[-1]} tokens, "
                                         f"{steps} steps, rows shuffled every step, "
                                         f"{joins} joins of {NP // 2}-token prompts"}


def roofline_of(model, shape, B, ctx, traffic_path):
    """Roofline object of the dominant decode kernel class (time per generated token), from
    HIP-event timings of back-to-back launches cycling through the layers."""
    prof = model.profile_kernels(B, iters=4 * shape.n_layers)
    kb = kernel_bytes(shape, B, ctx)
    per_token = {k: prof[k] * (shape.n_layers if k not in ("lmhead", "embed") else 1) for k in prof}
    dom = max(per_token, key=per_token.get)
    achieved = kb[dom] / (prof[dom] * 1e-6) / 1e9
    traffic = measured_traffic(traffic_path, dom) if traffic_path else None
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": dom, "avg_launch_us": round(prof[dom], 3), "bytes_per_launch": kb[dom],
            "per_kernel_us": {k: round(v, 3) for k, v in prof.items()},
            "per_token_us": {k: round(v, 1) for k, v in per_token.items()}}


def config_17b(args):
    """Qwen3-1.7B shape, 256-token prompts, 128 new tokens, B = 1 and 8: oracle-gated
    (quantization on two layers, B=1 prefill row + 2 steps teacher-forced, B=8 rows 0 and 7,
    free-running prefix of sequence 0), then timed."""
    import torch
    import int8_weight_only_amd as qd
    from workloads import SHAPES, make_weights, make_prompts
    shape = SHAPES["qwen3-1.7b"]
    NP, NN = 256, 128
    t = time.time()
    w = make_weights(shape, seed=0, gains="ones")
    log(f"[bench] 1.7B weights drawn in {time.time() - t:.1f}s")
    model = qd.Model(shape, w, max_batch=8, max_ctx=NP + NN, max_prefill_tokens=8 * NP)
    try:
        check_quantization(model, shape, w, (0, shape.n_layers - 1))
        runs = OracleRuns(shape, w)
        del w
        p8 = make_prompts(shape.vocab, NP, 8, seed0=1000)
        keys = [1000 + b for b in range(8)]
        par1 = rows_gate(model, runs, p8[:1], keys, [0], 2, "qwen3-1.7b")
        par8 = rows_gate(model, runs, p8, keys, [0, 7], 2, "qwen3-1.7b")
        out = {}
        for B, steps in ((1, 3), (8, 2)):
            _, pre, dec, _, res = time_generate(model, p8[:B], NN, steps, 1)
            dtok = B * (NN - 1) / (dec * 1e-6)
            out[f"decode_b{B}_tok_s"] = round(dtok, 1)
            out[f"decode_b{B}_hbm_frac"] = round(
                decode_bytes_per_step(shape, B, NP + (NN - 1) / 2.0) * dtok / B / 1e9 / PEAK_HBM_GBS, 4)
            out[f"prefill_b{B}_tok_s"] = round(B * NP / (pre * 1e-6), 1)
            n = free_run_gate(runs, keys[0], p8[0], res.generated[0], "qwen3-1.7b", 8)
            out[f"b{B}_seq0_oracle_prefix_steps"] = n
            log(f"[bench] 1.7B B={B}: decode {dtok:.1f} tok/s, prefill {B * NP / (pre * 1e-6):.0f} tok/s")
        out["parity_b1"] = par1
        out["parity_b8"] = par8
        out["workload"] = "qwen3-1.7b int8 greedy generate: 256-token prompts + 127 decode steps"
        return out
    finally:
        model.close()


def config_long(args, shape, w):
    """Qwen3-0.6B, 8192-token prompt, 2048 new tokens (KV cache to 10,239 positions), B=1.
    Oracle gate on a stated prefix: the first 2048 ids of the same prompt, prefill row + 2
    decode steps teacher-forced; the full-length run is checked by prefill-vs-decode
    consistency on the GPU.  Reports the attention share of the per-token time."""
    import torch
    import int8_weight_only_amd as qd
    from workloads import make_prompts
    NP, NN = 8192, 2048
    model = qd.Model(shape, w, max_batch=1, max_ctx=NP + NN, max_prefill_tokens=NP)
    try:
        prompt = make_prompts(shape.vocab, NP, 1, seed0=1000)[0]
        runs = OracleRuns(shape, w)
        par = rows_gate(model, runs, [prompt[:2048]], [1000], [0], 2, "qwen3-0.6b-2k")
        par["prefix"] = "first 2048 of the 8192 prompt ids"
        cons = consistency_gate(model, prompt, bar_for_config("qwen3-0.6b"))
        step_us, pre, dec, _, res = time_generate(model, [prompt], NN, 2, 1)
        dtok = (NN - 1) / (dec * 1e-6)
        mean_ctx = NP + (NN - 1) / 2.0
        prof = model.profile_kernels(1, iters=2 * shape.n_layers)
        attn_us = prof["attn"]
        per_tok = {k: prof[k] * (shape.n_layers if k not in ("lmhead", "embed") else 1) for k in prof}
        out = {"workload": "qwen3-0.6b int8 greedy generate: 8192-token prompt + 2047 decode steps",
               "decode_tok_s": round(dtok, 1),
               "decode_hbm_frac": round(decode_bytes_per_step(shape, 1, mean_ctx) * dtok / 1e9 / PEAK_HBM_GBS, 4),
               "prefill_tok_s": round(NP / (pre * 1e-6), 1),
               "prefill_mfma_frac": round(prefill_flops(shape, NP) / (pre * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "attn_us_per_layer_at_10k": round(attn_us, 3),
               "attn_share_of_kernel_time": round(attn_us * shape.n_layers / sum(per_tok.values()), 3),
               "per_kernel_us": {k: round(v, 3) for k, v in prof.items()},
               "parity_prefix": par, "parity_full_length": cons}
        log(f"[bench] long: decode {dtok:.1f} tok/s, prefill {NP / (pre * 1e-6):.0f} tok/s, "
            f"attention {attn_us:.2f} us/layer at ~10K positions")
        return out
    finally:
        model.close()


def bar_for_config(name):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import bar_for
    return bar_for(name)[0]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prompt", type=int, default=256)
    ap.add_argument("--new", type=int, default=128)
    ap.add_argument("--shape", default="qwen3-0.6b")
    ap.add_argument("--extra-batches", default="8,16,32",
                    help="batched decode lines measured after the main one ('' for none)")
    ap.add_argument("--no-extra", action="store_true", help="same as --extra-batches ''")
    ap.add_argument("--no-oracle", action="store_true", help="skip parity gate and CPU baseline")
    ap.add_argument("--no-continuous", action="store_true", help="skip the continuous-batching line")
    ap.add_argument("--no-sampled", action="store_true", help="skip the sampled-decode lines")
    ap.add_argument("--no-cache-timing", action="store_true", help="skip the load-cache line")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the Qwen3-1.7B and long-context (8192 + 2048) lines")
    ap.add_argument("--kernels-only", action="store_true",
                    help="no captured graphs and few dispatches: prefill prompt+new-2 tokens, "
                         "one decode step, then the per-kernel timing pass (for counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (to calibrate "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE against known bytes) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": n}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path is not "
              f"sharded across GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_weight_only_amd as qd
    from workloads import SHAPES, make_weights, make_prompts, make_prompt
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import bar_for

    shape = SHAPES[args.shape]
    B, NP, NN = args.batch, args.prompt, args.new
    ctx = NP + NN
    extras = [] if args.no_extra or not args.extra_batches else \
        [int(x) for x in args.extra_batches.split(",") if int(x) != B]
    max_batch = max([B] + extras)
    t = time.time()
    w = make_weights(shape, seed=0, gains="ones")
    log(f"[bench] weights drawn in {time.time() - t:.1f}s")
    t = time.time()
    model = qd.Model(shape, w, max_batch=max_batch, max_ctx=ctx,
                     max_prefill_tokens=max_batch * (NP + NN if args.kernels_only else NP))
    torch.cuda.synchronize()
    load_s = time.time() - t
    log(f"[bench] loaded + quantized on GPU in {load_s:.1f}s")
    prompts = make_prompts(shape.vocab, NP, max_batch, seed0=1000)
    keys = [1000 + b for b in range(max_batch)]

    if args.kernels_only:
        # same launch configuration as the timing pass below (context NP + NN - 1) with few
        # dispatches: prefill NP + NN - 2 tokens, one decode step, then the per-kernel pass
        long_prompts = make_prompts(shape.vocab, NP + NN - 2, B, seed0=1000)
        nxt, _ = model.prefill(list(long_prompts))
        model.decode_step(nxt)
        prof = model.profile_kernels(B, iters=4 * shape.n_layers)
        torch.cuda.synchronize()
        print(json.dumps({"kernels_only": True, "per_kernel_us": prof}), flush=True)
        model.close()
        return

    oracle = not args.no_oracle and NP <= 1024 and args.shape in ("qwen3-0.6b", "qwen3-1.7b")
    parity, cpu, runs = {"checked": False}, None, None
    if oracle:
        n_q = check_quantization(model, shape, w, (0, shape.n_layers - 1))
        runs = OracleRuns(shape, w)
        parity = rows_gate(model, runs, prompts[:B], keys, list(range(B)) if B <= 2 else [0, B - 1],
                           2, args.shape)
        parity["quantized_matrices_bit_exact"] = n_q
        log(f"[bench] parity ok: {parity}")

    load_line = {}
    if not args.no_cache_timing:
        load_line = time_cache_load(model, shape, max_batch, ctx, NP, load_s)
    step_us, pre_us, dec_us, wall, res = time_generate(model, prompts[:B], NN, args.steps, args.warmup)
    value = B * NN / (step_us * 1e-6)
    decode_tok_s = B * (NN - 1) / (dec_us * 1e-6)
    prefill_tok_s = B * NP / (pre_us * 1e-6)
    mean_ctx = NP + (NN - 1) / 2.0
    hbm = decode_bytes_per_step(shape, B, mean_ctx) * decode_tok_s / B / 1e9 / PEAK_HBM_GBS
    log(f"[bench] B={B}: {value:.1f} tok/s whole call, decode {decode_tok_s:.1f} tok/s "
        f"({hbm * 100:.2f}% HBM), prefill {prefill_tok_s:.0f} tok/s, wall/step {wall * 1e3:.2f} ms")
    if oracle:
        parity["free_run_oracle_prefix_steps"] = free_run_gate(runs, keys[0], prompts[0],
                                                               res.generated[0], args.shape)

    tpath = os.path.join(ROOT, "profiles", f"decode_b{B}_{args.shape}_traffic.md") \
        if (NP, NN) == (256, 128) else None
    roofline = roofline_of(model, shape, B, ctx - 1, tpath)
    log(f"[bench] kernel us: {roofline['per_kernel_us']}")

    extra = {}
    for xb in extras:
        bprompts = prompts[:xb]
        if oracle:
            extra[f"decode_b{xb}_parity"] = rows_gate(model, runs, bprompts, keys, [0, xb - 1], 2,
                                                      args.shape)
        _, xpre, xdec, _, xr = time_generate(model, bprompts, NN, 2, 1)
        dtok = xb * (NN - 1) / (xdec * 1e-6)
        extra[f"decode_b{xb}_tok_s"] = round(dtok, 1)
        extra[f"decode_b{xb}_hbm_frac"] = round(
            decode_bytes_per_step(shape, xb, mean_ctx) * dtok / xb / 1e9 / PEAK_HBM_GBS, 4)
        extra[f"prefill_b{xb}_tok_s"] = round(xb * NP / (xpre * 1e-6), 1)
        extra[f"b{xb}_over_b{B}"] = round(dtok / decode_tok_s, 2)
        if oracle:
            extra[f"b{xb}_seq0_oracle_prefix_steps"] = free_run_gate(
                runs, keys[0], prompts[0], xr.generated[0], args.shape)
        log(f"[bench] B={xb}: decode {dtok:.1f} tok/s, prefill {xb * NP / (xpre * 1e-6):.0f} tok/s")

    if extras and max(extras) >= 8 and not args.no_continuous:
        S = max(extras)
        if oracle:
            # slot-addressed prefill of two prompts, then decode steps listing their slots in a
            # fresh random order each step, against each prompt's own oracle run
            cp = [make_prompt(shape.vocab, NP // 2 + 40, 3001), make_prompt(shape.vocab, NP // 2, 3002)]
            extra["continuous_parity"] = rows_gate(model, runs, cp, [3001, 3002], [0, 1], 2,
                                                   args.shape, slots=[S - 3, 5])
        extra.update(time_continuous(model, shape, S, NP, NN))
    if not args.no_sampled:
        for sb in sorted({B} | ({max(extras)} if extras else set())):
            if oracle:
                extra[f"sampled_b{sb}_parity"] = sampled_gate(
                    model, shape, sb, NP, [1234 + b for b in range(sb)], SAMPLED)
            extra.update(time_sampled(model, shape, sb, NP, NN))

    if oracle:
        cpu_model, blas = cpu_info()
        runs.get(keys[0], prompts[0], NN)   # the workload's own 127 decode steps on the CPU
        cpu = {"value": round(runs.n_dec / runs.t_dec, 3), "unit": "tok/s",
               "cores": blas or int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0)))),
               "kind": "oracle", "cpu_model": cpu_model, "blas_threads": blas,
               "sample": f"the oracle runs of this benchmark's parity gates on {args.shape}: "
                         f"{runs.n_pre} prompt tokens prefilled in {runs.t_pre:.1f} s "
                         f"({runs.n_pre / max(runs.t_pre, 1e-9):.1f} tok/s), {runs.n_dec} greedy "
                         f"decode steps at B=1 in {runs.t_dec:.1f} s; value = decode steps / "
                         f"their wall time"}
    model.close()

    configs = {}
    if not args.no_configs and args.shape == "qwen3-0.6b" and (NP, NN, B) == (256, 128, 1) and oracle:
        configs["qwen3_1.7b"] = config_17b(args)
        configs["long_8192_2048"] = config_long(args, shape, w)
    del w

    pf = prefill_flops(shape, NP)
    line = {
        "metric": "int8 decode tok/s + % HBM roofline, Qwen3-0.6B shape, B=1/32; prefill tok/s",
        "value": round(value, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_us / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8xbf16",
        "data": "synthetic",
        "config": {"workload": f"{args.shape} int8 greedy generate: B={B}, {NP}-token prompt "
                               f"prefill + {NN - 1} decode steps ({NN} new tokens)",
                   "global_batch": B, "seq_len": ctx, "parallelism": "none (1 GPU)",
                   "weights": "random-init N(0,0.02^2) seed 0, int8 per output channel",
                   "prompts": "uniform ids, seed 1000+b"},
        "value_counts": "generated tokens / (prefill + decode) device time of one call",
        "decode_tok_s": round(decode_tok_s, 1),
        "decode_hbm_frac": round(hbm, 4),
        "prefill_tok_s": round(prefill_tok_s, 1),
        "prefill_mfma_frac": round(pf * prefill_tok_s / NP / 1e12 / PEAK_BF16_TFLOPS, 4),
        "wall_ms_per_step_incl_host": round(wall * 1e3, 4),
        **extra,
        **load_line,
        **configs,
        "parity": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
