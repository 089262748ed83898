"""Independent float64 brute-force forward pass, used only to pin the oracle.

Written separately from the oracle on purpose, in a different form:
* no KV cache: every call recomputes the whole sequence from the token ids;
* key/value heads are explicitly repeated to the query-head count;
* RoPE is a complex multiplication z * exp(i * p * w) on (x_i, x_{i+D/2}) pairs;
* causal masking puts -inf above the diagonal of the full score matrix.
It takes dequantized float64 weights (code times row scale) and performs no
rounding anywhere, so it must agree with the oracle's exact mode to float64
round-off.  The architecture follows "Model-agnostic LLM inference", section
"Supported models".
"""
from __future__ import annotations

import numpy as np


def dequantized(qmodel: dict) -> dict:
    """float64 weights from int8 codes and fp32 row scales."""
    dq = lambda qs: qs[0].astype(np.float64) * qs[1].astype(np.float64)[:, None]
    out = {"embed": dq(qmodel["embed"]), "final_norm": qmodel["final_norm"].astype(np.float64),
           "layers": []}
    for L in qmodel["layers"]:
        d = {m: dq(L[m]) for m in ("q", "k", "v", "o", "gate", "up", "down")}
        for g in ("in_norm", "post_norm", "q_norm", "k_norm"):
            d[g] = L[g].astype(np.float64)
        out["layers"].append(d)
    return out


def _norm(x, g, eps):
    return x * (1.0 / np.sqrt(np.mean(x ** 2, axis=-1, keepdims=True) + eps)) * g


def _rope_complex(x, theta):
    # x: [T, heads, D]; rotate pairs (i, i + D/2) by angle p * theta^(-2i/D)
    T, nh, D = x.shape
    half = D // 2
    w = np.power(float(theta), -np.arange(half) * 2.0 / D)
    p = np.arange(T)[:, None, None]
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * p * w[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def logits_all(shape, W: dict, ids) -> np.ndarray:
    """Logits [T, V] at every position of the token sequence ``ids``."""
    H, KV, D, eps = shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps
    ids = np.asarray(ids, dtype=np.int64)
    T = ids.size
    x = W["embed"][ids].copy()
    mask = np.triu(np.full((T, T), -np.inf), k=1)
    for L in W["layers"]:
        a = _norm(x, L["in_norm"], eps)
        Q = (a @ L["q"].T).reshape(T, H, D)
        K = (a @ L["k"].T).reshape(T, KV, D)
        V = (a @ L["v"].T).reshape(T, KV, D)
        Q = _rope_complex(_norm(Q, L["q_norm"], eps), shape.rope_theta)
        K = _rope_complex(_norm(K, L["k_norm"], eps), shape.rope_theta)
        K = np.repeat(K, H // KV, axis=1)
        V = np.repeat(V, H // KV, axis=1)
        S = np.einsum("thd,shd->hts", Q, K) / np.sqrt(D) + mask[None]
        S = np.exp(S - S.max(axis=-1, keepdims=True))
        P = S / S.sum(axis=-1, keepdims=True)
        O = np.einsum("hts,shd->thd", P, V).reshape(T, H * D)
        x = x + O @ L["o"].T
        b = _norm(x, L["post_norm"], eps)
        g = b @ L["gate"].T
        u = b @ L["up"].T
        x = x + ((g / (1.0 + np.exp(-g))) * u) @ L["down"].T
    f = _norm(x, W["final_norm"], eps)
    return f @ W["embed"].T


def greedy(shape, W: dict, prompt, n_new: int):
    """Greedy ids and per-step logits by full recomputation at every step."""
    seq = list(int(t) for t in prompt)
    ids, steps = [], []
    for _ in range(n_new):
        lg = logits_all(shape, W, seq)[-1]
        t = int(np.argmax(lg))
        ids.append(t)
        steps.append(lg)
        seq.append(t)
    return np.array(ids), np.stack(steps)
