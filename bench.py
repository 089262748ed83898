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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prompt", type=int, default=256)
    ap.add_argument("--new", type=int, default=128)
    ap.add_argument("--shape", default="qwen3-0.6b")
    ap.add_argument("--no-extra", action="store_true", help="skip the B=32 line")
    ap.add_argument("--no-oracle", action="store_true", help="skip parity gate and CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path is not "
              f"sharded across GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_weight_only_amd as qd
    from workloads import SHAPES, make_weights, make_prompts

    shape = SHAPES[args.shape]
    B, NP, NN = args.batch, args.prompt, args.new
    ctx = NP + NN
    extra_B = 32
    max_batch = max(B, 1 if args.no_extra else extra_B)
    t = time.time()
    w = make_weights(shape, seed=0, gains="ones")
    log(f"[bench] weights drawn in {time.time() - t:.1f}s")
    t = time.time()
    model = qd.Model(shape, w, max_batch=max_batch, max_ctx=ctx,
                     max_prefill_tokens=max_batch * NP)
    torch.cuda.synchronize()
    log(f"[bench] loaded + quantized on GPU in {time.time() - t:.1f}s")
    prompts = make_prompts(shape.vocab, NP, B, seed0=1000)

    # ---- parity gate (sampled, full size) and CPU baseline ----
    parity = {"checked": False}
    cpu = None
    if not args.no_oracle:
        from oracle import Oracle, quantize_rows, quantize_model
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import bar_for, logit_err
        t = time.time()
        samples = [("embed", 0)] + [(m, l) for l in (0, shape.n_layers - 1)
                                    for m in ("q", "k", "v", "o", "gate", "up", "down")]
        for name, layer in samples:
            q, s = model.export_quantized(name, layer)
            src = w["embed"] if name == "embed" else w["layers"][layer][name]
            qr, sr = quantize_rows(src)
            if not (np.array_equal(q, qr) and np.array_equal(s, sr)):
                raise SystemExit(f"parity gate failed: quantized {name}[{layer}] differs")
        log(f"[bench] quantization bit-exact on {len(samples)} matrices ({time.time() - t:.1f}s)")
        t = time.time()
        qm = quantize_model(w)
        orc = Oracle(shape, qm, mode="bf16")
        log(f"[bench] oracle ready in {time.time() - t:.1f}s")
        n_chk = 3
        seq = orc.new_sequence()
        t0 = time.time()
        ol = [orc.forward(seq, prompts[0])]
        t_pre = time.time() - t0
        oids = [int(np.argmax(ol[0]))]
        t0 = time.time()
        for k in range(1, n_chk):
            ol.append(orc.forward(seq, [oids[-1]]))
            oids.append(int(np.argmax(ol[-1])))
        t_dec = time.time() - t0
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        cpu = {"value": round((n_chk - 1) / t_dec, 3), "unit": "tok/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{args.shape} B=1: one {NP}-token prompt prefilled "
                         f"({NP / t_pre:.1f} tok/s), then {n_chk - 1} greedy decode steps; "
                         f"value = decode steps / their wall time"}
        nxt, lg = model.prefill([prompts[0]], logits=True)
        errs = [logit_err(lg[0].cpu().numpy(), ol[0])]
        ids_ok = int(nxt[0].item()) == int(np.argmax(lg[0].cpu().numpy()))
        for k in range(1, n_chk):
            feed = torch.tensor([oids[k - 1]], dtype=torch.int32, device="cuda")
            nxt, lg = model.decode_step(feed, logits=True)
            errs.append(logit_err(lg[0].cpu().numpy(), ol[k]))
            ids_ok &= int(nxt[0].item()) == int(np.argmax(lg[0].cpu().numpy()))
        bar, _ = bar_for(args.shape) if args.shape in ("qwen3-0.6b",) else (2e-2, None)
        parity = {"checked": True, "steps": n_chk, "max_logit_err": round(max(errs), 5),
                  "bar": bar, "fused_argmax_exact": bool(ids_ok)}
        if max(errs) > bar or not ids_ok:
            raise SystemExit(f"parity gate failed: {parity}")
        log(f"[bench] parity ok: {parity}")
        del qm, orc, seq

    # ---- timed region: K generate calls at B ----
    for _ in range(args.warmup):
        model.generate_greedy(list(prompts), NN)
    torch.cuda.synchronize()
    dev_us, pre_us, dec_us = [], [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r = model.generate_greedy(list(prompts), NN)
        dev_us.append(r.prefill_us + r.decode_us)
        pre_us.append(r.prefill_us)
        dec_us.append(r.decode_us)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = float(np.mean(dev_us))
    value = B * NN / (step_us * 1e-6)
    decode_tok_s = B * (NN - 1) / (np.mean(dec_us) * 1e-6)
    prefill_tok_s = B * NP / (np.mean(pre_us) * 1e-6)
    mean_ctx = NP + (NN - 1) / 2.0
    hbm_b1 = decode_bytes_per_step(shape, B, mean_ctx) * decode_tok_s / B / 1e9 / PEAK_HBM_GBS
    log(f"[bench] B={B}: {value:.1f} tok/s whole call, decode {decode_tok_s:.1f} tok/s, "
        f"prefill {prefill_tok_s:.0f} tok/s, wall/step {wall / args.steps * 1e3:.2f} ms")

    # ---- roofline of the dominant decode kernel (HIP events, live) ----
    prof = model.profile_kernels(B, iters=100)
    kb = kernel_bytes(shape, B, ctx - 1)
    per_token = {k: prof[k] * (shape.n_layers if k not in ("lmhead", "embed") else 1) for k in prof}
    dom = max(per_token, key=per_token.get)
    achieved = kb[dom] / (prof[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": dom, "avg_launch_us": round(prof[dom], 3),
                "bytes_per_launch": kb[dom],
                "per_kernel_us": {k: round(v, 3) for k, v in prof.items()}}
    log(f"[bench] kernel us: {roofline['per_kernel_us']}")

    extra = {}
    if not args.no_extra:
        bprompts = make_prompts(shape.vocab, NP, extra_B, seed0=1000)
        model.generate_greedy(list(bprompts), NN)
        rs = [model.generate_greedy(list(bprompts), NN) for _ in range(2)]
        # batch independence: sequence 0 of the batch equals the B=1 run of the same prompt
        same = np.array_equal(rs[0].generated[0], r.generated[0]) if B == 1 else None
        dec32 = extra_B * (NN - 1) / (np.mean([x.decode_us for x in rs]) * 1e-6)
        pre32 = extra_B * NP / (np.mean([x.prefill_us for x in rs]) * 1e-6)
        extra = {"decode_b32_tok_s": round(dec32, 1),
                 "decode_b32_hbm_frac": round(decode_bytes_per_step(shape, extra_B, mean_ctx)
                                              * dec32 / extra_B / 1e9 / PEAK_HBM_GBS, 4),
                 "prefill_b32_tok_s": round(pre32, 1),
                 "b32_over_b1": round(dec32 / decode_tok_s, 2),
                 "b32_seq0_equals_b1": same}
        log(f"[bench] B=32 decode {dec32:.1f} tok/s, prefill {pre32:.0f} tok/s")

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
        "decode_tok_s": round(decode_tok_s, 1),
        "decode_hbm_frac": round(hbm_b1, 4),
        "prefill_tok_s": round(prefill_tok_s, 1),
        "prefill_mfma_frac": round(pf * prefill_tok_s / NP / 1e12 / PEAK_BF16_TFLOPS, 4),
        "wall_ms_per_step_incl_host": round(wall / args.steps * 1e3, 4),
        **extra,
        "parity": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    model.close()


if __name__ == "__main__":
    main()
