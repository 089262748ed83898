"""Writes tests/golden/noise_floor.json: how far apart two valid implementations of the
bf16 precision contract land, measured with the CPU oracle alone.

The contract rounds every activation to bf16.  An implementation that accumulates in
fp32 (in any order) instead of float64 reaches each rounding point with a relative
difference of about 1e-7; whenever that flips one bf16 rounding, the flipped element
perturbs every value computed from it, which flips further roundings downstream.
Through several layers the two runs decorrelate down to the bf16 rounding noise of the
whole network.  This script measures that spread: the oracle against copies of itself
whose every bf16 rounding point sees a uniform relative perturbation of +-6e-8 (three
perturbation seeds), teacher-forced on the same ids, as max |dlogit| / RMS(logits) per
step.  It calls nothing but ``oracle/`` and ``workloads``.

The parity bar used by the tests is max(2e-2, 1.5 * floor): 2e-2 is the stated
tolerance; where the contract's own spread exceeds it, no bf16 implementation can do
better than the spread, and 1.5x leaves room for the max over the vocabulary.

Usage: python tests/golden/make_noise_floor.py [config ...]
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import Oracle, quantize_model, bf16  # noqa: E402
from workloads import SHAPES, ModelShape, make_weights, make_prompt  # noqa: E402

CONFIGS = {
    # name: (shape, weight seed, gains, prompt length, prompt seed, steps)
    "tiny": (SHAPES["tiny"], 0, "uniform", 16, 1000, 16),
    "tiny-b": (SHAPES["tiny"], 2, "uniform", 12, 2000, 6),
    "wide": (ModelShape(hidden=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=64,
                        intermediate=256, vocab=512), 1, "uniform", 77, 1001, 12),
    "odd": (ModelShape(hidden=96, n_layers=3, n_heads=6, n_kv_heads=2, head_dim=32,
                       intermediate=160, vocab=1000), 1, "uniform", 77, 1001, 12),
    "mid": (ModelShape(hidden=512, n_layers=2, n_heads=8, n_kv_heads=4, head_dim=128,
                       intermediate=1024, vocab=4096), 4, "uniform", 200, 1004, 8),
    # hidden and intermediate not multiples of 128 (ragged 128-k blocks in split-K)
    "splitk": (ModelShape(hidden=288, n_layers=2, n_heads=6, n_kv_heads=2, head_dim=32,
                          intermediate=544, vocab=1000), 5, "uniform", 8, 4000, 4),
    # long context at a small shape: many attention splits and prefill tiles
    "wide-long": (ModelShape(hidden=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=64,
                             intermediate=256, vocab=512), 5, "uniform", 1500, 1005, 24),
    "qwen3-0.6b": (SHAPES["qwen3-0.6b"], 0, "ones", 256, 1000, 4),
    # every dimension of Qwen3-0.6B but 2 layers: the kernel instantiations of the full
    # model (they depend on the widths, heads and vocabulary, not on the depth)
    "qwen3-0.6b-l2": (ModelShape(hidden=1024, n_layers=2, n_heads=16, n_kv_heads=8,
                                 head_dim=128, intermediate=3072, vocab=151936),
                      0, "uniform", 256, 1000, 5),
    # the same with an 8192-token prompt: decode attention over > 8 merged splits at D=128
    "long-0.6b-l2": (ModelShape(hidden=1024, n_layers=2, n_heads=16, n_kv_heads=8,
                                head_dim=128, intermediate=3072, vocab=151936),
                     0, "uniform", 8192, 1005, 4),
    # head_dim 64 with 32 heads of q|k|v and a 2048-token prompt: the prefill q|k|v GEMM
    # takes 256 tiles of 128x128 (two heads each) with QK-norm and RoPE in its epilogue
    "rope64": (ModelShape(hidden=256, n_layers=2, n_heads=16, n_kv_heads=8, head_dim=64,
                          intermediate=512, vocab=1000), 6, "uniform", 2048, 1006, 3),
    "qwen3-1.7b": (SHAPES["qwen3-1.7b"], 0, "ones", 256, 1000, 3),
    # Qwen3-0.6B on the first 2048 ids of the long-context prompt (8192 ids, seed 1000)
    "qwen3-0.6b-2k": (SHAPES["qwen3-0.6b"], 0, "ones", 2048, 1000, 3),
}
PERT = 6e-8
FACTOR = 1.5
STRICT = 2e-2


class _Perturbed(Oracle):
    def __init__(self, *a, seed=0, **k):
        super().__init__(*a, **k)
        rng = np.random.default_rng(seed)
        self._act = lambda v: bf16(np.asarray(v) * (1.0 + rng.uniform(-1, 1, np.shape(v)) * PERT))


def measure(name):
    shape, wseed, gains, n_prompt, pseed, steps = CONFIGS[name]
    qm = quantize_model(make_weights(shape, seed=wseed, gains=gains))
    prompt = make_prompt(shape.vocab, n_prompt, pseed)
    ref = Oracle(shape, qm).generate(prompt, steps)
    per_step = np.zeros(steps)
    for s in range(3):
        alt = _Perturbed(shape, qm, seed=s).generate(prompt, steps, teacher=ref["ids"])
        for k in range(steps):
            lr = ref["logits"][k]
            e = np.max(np.abs(alt["logits"][k] - lr)) / np.sqrt(np.mean(lr * lr))
            per_step[k] = max(per_step[k], e)
    floor = float(per_step.max())
    rms = float(np.sqrt(np.mean(ref["logits"] ** 2)))
    bar = max(STRICT, FACTOR * floor)
    return {"floor": round(floor, 5), "per_step": [round(float(x), 5) for x in per_step],
            "bar": round(bar, 5), "logit_rms": round(rms, 5),
            "margin_gate": round(max(5e-2, 2 * bar * rms), 5),
            "recipe": {"weight_seed": wseed, "gains": gains, "prompt_len": n_prompt,
                       "prompt_seed": pseed, "steps": steps, "perturbation": PERT,
                       "perturbation_seeds": [0, 1, 2]}}


def main(names):
    path = os.path.join(HERE, "noise_floor.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    for n in names or list(CONFIGS):
        data[n] = measure(n)
        print(n, data[n]["floor"], data[n]["bar"], flush=True)
        json.dump(data, open(path, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
