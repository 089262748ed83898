"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module draws numbers and nothing else: it holds none of the decoder's
arithmetic (no quantization, no normalization, no matmul).  Both sides of every
parity test take their weights and prompts from here, so the oracle and the HIP
path see the same bytes.

Model shapes follow the Qwen3 decoder family described on "Model-agnostic LLM
inference" (section "Supported models") and the fixed Qwen3-0.6B-Base shape on
"Run local LLM decode" (section "Limitations").  Weights are random-init with a
normal of standard deviation 0.02 (read as N(0, 0.02^2)); prompts are uniform
token ids.  Real checkpoints and real prompts are not available, so these stand
in for them at the same shapes and sizes.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

__all__ = [
    "ModelShape", "SHAPES", "make_weights", "make_prompt", "make_prompts",
    "weight_names", "layer_matrix_shapes",
]


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Decoder dimensions, named after the checkpoint ``config.json`` fields."""
    hidden: int            # hidden_size
    n_layers: int          # num_hidden_layers
    n_heads: int           # num_attention_heads
    n_kv_heads: int        # num_key_value_heads
    head_dim: int          # head_dim
    intermediate: int      # intermediate_size
    vocab: int             # vocab_size
    rms_eps: float = 1e-6  # rms_norm_eps
    rope_theta: float = 1e6
    tie_word_embeddings: bool = True
    attention_bias: bool = False


SHAPES = {
    # small decoder used for parity checks the oracle finishes in seconds
    "tiny": ModelShape(hidden=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=32,
                       intermediate=384, vocab=1024),
    # Qwen3-0.6B-Base
    "qwen3-0.6b": ModelShape(hidden=1024, n_layers=28, n_heads=16, n_kv_heads=8, head_dim=128,
                             intermediate=3072, vocab=151936),
    # Qwen3-1.7B
    "qwen3-1.7b": ModelShape(hidden=2048, n_layers=28, n_heads=16, n_kv_heads=8, head_dim=128,
                             intermediate=6144, vocab=151936),
}

LAYER_MATRICES = ("q", "k", "v", "o", "gate", "up", "down")
LAYER_GAINS = ("in_norm", "post_norm", "q_norm", "k_norm")

# Elements per independent random stream.  Fixed, so the values do not depend on
# how many threads draw them.
_CHUNK = 1 << 22


def layer_matrix_shapes(s: ModelShape) -> dict:
    """[out, in] shape of every per-layer projection (row = output channel)."""
    qd = s.n_heads * s.head_dim
    kvd = s.n_kv_heads * s.head_dim
    return {
        "q": (qd, s.hidden), "k": (kvd, s.hidden), "v": (kvd, s.hidden),
        "o": (s.hidden, qd),
        "gate": (s.intermediate, s.hidden), "up": (s.intermediate, s.hidden),
        "down": (s.hidden, s.intermediate),
    }


def weight_names(s: ModelShape):
    """Draw order of the random matrices: embedding, then per layer q,k,v,o,gate,up,down."""
    names = [("embed", (s.vocab, s.hidden))]
    shp = layer_matrix_shapes(s)
    for li in range(s.n_layers):
        for m in LAYER_MATRICES:
            names.append((f"layers.{li}.{m}", shp[m]))
    return names


def _normal_fill(out: np.ndarray, seed_seq: np.random.SeedSequence, std: float, threads: int):
    flat = out.reshape(-1)
    n_chunks = (flat.size + _CHUNK - 1) // _CHUNK
    seqs = seed_seq.spawn(n_chunks)

    def fill(i):
        part = flat[i * _CHUNK:(i + 1) * _CHUNK]
        np.random.default_rng(seqs[i]).standard_normal(out=part, dtype=np.float32)
        part *= np.float32(std)

    if threads <= 1 or n_chunks == 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n_chunks)))


def make_weights(shape: ModelShape, seed: int = 0, gains: str = "ones", std: float = 0.02,
                 threads: int | None = None) -> dict:
    """fp32 weights in checkpoint layout ([out, in] row-major), drawn from ``seed``.

    Returns ``{"embed": [V,d], "final_norm": [d], "layers": [ {q,k,v,o,gate,up,down,
    in_norm, post_norm, q_norm, k_norm}, ... ]}``.

    gains="ones" sets every norm gain to 1.0 (standard init); gains="uniform" draws
    them from U(0.5, 1.5) so a dropped gain multiply shows up in a comparison.
    """
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    root = np.random.SeedSequence(seed)
    names = weight_names(shape)
    mats_seq = root.spawn(len(names) + 1)
    out = {"layers": [dict() for _ in range(shape.n_layers)]}
    for (name, shp), ss in zip(names, mats_seq[:-1]):
        arr = np.empty(shp, dtype=np.float32)
        _normal_fill(arr, ss, std, threads)
        if name == "embed":
            out["embed"] = arr
        else:
            _, li, m = name.split(".")
            out["layers"][int(li)][m] = arr
    grng = np.random.default_rng(mats_seq[-1])

    def gain(n):
        if gains == "ones":
            return np.ones(n, dtype=np.float32)
        if gains == "uniform":
            return grng.uniform(0.5, 1.5, n).astype(np.float32)
        raise ValueError(f"unknown gains mode {gains!r}")

    for L in out["layers"]:
        L["in_norm"] = gain(shape.hidden)
        L["post_norm"] = gain(shape.hidden)
        L["q_norm"] = gain(shape.head_dim)
        L["k_norm"] = gain(shape.head_dim)
    out["final_norm"] = gain(shape.hidden)
    return out


def make_prompt(vocab: int, n: int, seed: int) -> np.ndarray:
    """``n`` token ids uniform over [0, vocab), int32."""
    return np.random.default_rng(seed).integers(0, vocab, n).astype(np.int32)


def make_prompts(vocab: int, n: int, batch: int, seed0: int = 1000) -> np.ndarray:
    """``batch`` prompts of ``n`` ids; sequence b uses seed ``seed0 + b``.  [batch, n] int32."""
    return np.stack([make_prompt(vocab, n, seed0 + b) for b in range(batch)])
