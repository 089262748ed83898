"""CPU oracle for the int8 weight-only Qwen3 decoder step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

What it computes, and where each step comes from:

* The decoder: grouped-query attention with RMSNorm on Q and K, RoPE, a
  SiLU-gated feed-forward block, tied input/output embeddings and no attention
  bias ("Model-agnostic LLM inference", section "Supported models"; the
  Qwen3-0.6B-Base dimensions in "Run local LLM decode", section "Limitations").
* Weights are stored as int8 with one scale per output row ("Model-agnostic LLM
  inference", section "The quantized load cache").  The pages leave the scheme
  open; the precision contract used here is: symmetric per-output-channel int8
  with fp32 scales (absmax / 127, round-half-to-even, IEEE fp32 division), bf16
  activations, fp32-or-better accumulation, fp32 RMSNorm and softmax, a bf16 KV
  cache and fp32 logits.
* Prefill reads the whole prompt and fills the KV cache; decode produces one
  token per step; greedy selection takes the arg-max of the logits on every
  step, generating up to ``max_new_tokens`` ("LLM inference overview", section
  "Results"; "Model-agnostic LLM inference", section "Notes").

Arithmetic is float64 throughout.  In ``mode="bf16"`` every activation tensor the
model materializes is rounded to bf16 (through fp32) and logits to fp32; in
``mode="exact"`` no rounding happens at all (the weights are still the int8 codes
times their scales).  The quantizer itself is always fp32, because its result is
an integer code that must be bit-exact.

Readings of points the pages leave open (each also listed in the design notes):
rotate-half RoPE pairing (x_i, x_{i+D/2}) with inv_freq_i = theta^(-2i/D);
QK-norm per head over head_dim with one shared gain, before RoPE; query head h
uses KV head h // (H / KV); attention scale 1/sqrt(head_dim); pre-norm residual
blocks and a final RMSNorm; LM head = embedding matrix (tied); arg-max ties go
to the lowest index.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16", "quantize_rows", "quantize_model", "Oracle", "greedy_argmax",
    "packed_weight_bytes",
]


# --------------------------------------------------------------------------------------
# rounding helpers

def bf16(x) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even), returned as float64.

    The value is first rounded to fp32, as a GPU holding an fp32 register would,
    and then its low 16 mantissa bits are rounded away.
    """
    f = np.asarray(x, dtype=np.float32)
    if np.isnan(f).any():
        raise FloatingPointError("NaN reached a bf16 rounding point")
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def fp32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# quantization (load time)

def quantize_rows(w: np.ndarray):
    """Symmetric per-row int8 quantization of an fp32 [rows, cols] matrix.

    For each row r: a = max |w_r|;  s_r = fp32(a / 127);  q = clamp(rint(fp32(w / s_r)),
    -127, 127).  A row of zeros gets s = 0 and q = 0.  All divisions are IEEE fp32
    (correctly rounded); rint is round-half-to-even.
    Returns (q int8 [rows, cols], s fp32 [rows]).
    """
    w = np.asarray(w, dtype=np.float32)
    a = np.max(np.abs(w), axis=1)
    s = (a / np.float32(127.0)).astype(np.float32)
    zero = s == 0
    safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
    ratio = (w / safe[:, None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -127, 127).astype(np.int8)
    q[zero] = 0
    return q, s


def quantize_model(weights: dict) -> dict:
    """Quantize every projection and the (tied) embedding; gains stay fp32."""
    qm = {"layers": []}
    qm["embed"] = quantize_rows(weights["embed"])
    for L in weights["layers"]:
        d = {}
        for m in ("q", "k", "v", "o", "gate", "up", "down"):
            d[m] = quantize_rows(L[m])
        for g in ("in_norm", "post_norm", "q_norm", "k_norm"):
            d[g] = np.asarray(L[g], dtype=np.float32)
        qm["layers"].append(d)
    qm["final_norm"] = np.asarray(weights["final_norm"], dtype=np.float32)
    return qm


def packed_weight_bytes(shape) -> int:
    """Bytes of the quantized model: int8 codes, one fp32 scale per row, fp32 gains,
    the tied embedding stored once."""
    d, H, KV, D, I, V, L = (shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                            shape.intermediate, shape.vocab, shape.n_layers)
    rows_cols = [(H * D, d), (KV * D, d), (KV * D, d), (d, H * D), (I, d), (I, d), (d, I)]
    per_layer = sum(r * c + 4 * r for r, c in rows_cols) + 4 * (2 * d + 2 * D)
    return L * per_layer + (V * d + 4 * V) + 4 * d


# --------------------------------------------------------------------------------------
# the forward pass

def greedy_argmax(logits: np.ndarray) -> int:
    """Index of the largest logit, lowest index among ties (-0.0 equals +0.0)."""
    logits = np.asarray(logits)
    if np.isnan(logits).any():
        raise FloatingPointError("NaN logit")
    return int(np.argmax(logits))


class _Seq:
    """Per-sequence KV cache: K and V per layer as [n_kv_heads, positions, head_dim]."""

    def __init__(self, n_layers, n_kv, D):
        self.k = [np.zeros((n_kv, 0, D)) for _ in range(n_layers)]
        self.v = [np.zeros((n_kv, 0, D)) for _ in range(n_layers)]
        self.length = 0


class Oracle:
    """Plain CPU forward pass of the quantized decoder, one sequence at a time."""

    def __init__(self, shape, qmodel: dict, mode: str = "bf16"):
        if mode not in ("bf16", "exact"):
            raise ValueError(mode)
        self.shape = shape
        self.mode = mode
        self._act = bf16 if mode == "bf16" else (lambda a: np.asarray(a, dtype=np.float64))
        self._logit = fp32 if mode == "bf16" else (lambda a: np.asarray(a, dtype=np.float64))
        # codes as float64 (exact) for the matmuls, scales as float64 (exact)
        self.E_q = qmodel["embed"][0].astype(np.float64)
        self.E_q8 = qmodel["embed"][0]
        self.E_s = qmodel["embed"][1].astype(np.float64)
        self.E_s32 = qmodel["embed"][1]
        self.layers = []
        for L in qmodel["layers"]:
            d = {}
            for m in ("q", "k", "v", "o", "gate", "up", "down"):
                d[m] = (L[m][0].astype(np.float64), L[m][1].astype(np.float64))
            for g in ("in_norm", "post_norm", "q_norm", "k_norm"):
                d[g] = L[g].astype(np.float64)
            self.layers.append(d)
        self.final_norm = qmodel["final_norm"].astype(np.float64)
        D = shape.head_dim
        i = np.arange(D // 2, dtype=np.float64)
        self.inv_freq = float(shape.rope_theta) ** (-2.0 * i / D)

    # ---- building blocks ------------------------------------------------------------

    def new_sequence(self) -> _Seq:
        s = self.shape
        return _Seq(s.n_layers, s.n_kv_heads, s.head_dim)

    def embed(self, ids):
        """Row t of the tied embedding, dequantized: code times row scale in fp32."""
        ids = np.asarray(ids)
        if self.mode == "bf16":
            prod = self.E_q8[ids].astype(np.float32) * self.E_s32[ids][:, None]
            return bf16(prod)
        return self.E_q[ids] * self.E_s[ids][:, None]

    def rmsnorm(self, y, g):
        """y / sqrt(mean(y^2) + eps) * g over the last axis."""
        ms = np.mean(y * y, axis=-1, keepdims=True)
        return self._act(y / np.sqrt(ms + self.shape.rms_eps) * g)

    def proj(self, W, y):
        """Dequantizing projection: per output row, (sum_k code[n,k] * y[k]) * scale[n]."""
        q, s = W
        return self._act((y @ q.T) * s)

    def rope(self, x, positions):
        """Rotate-half RoPE.  x: [rows, heads, D], positions: [rows]."""
        D = self.shape.head_dim
        h = D // 2
        ang = np.asarray(positions, dtype=np.float64)[:, None] * self.inv_freq[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        x1 = x[..., :h]
        x2 = x[..., h:]
        out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
        return self._act(out)

    def attention(self, q, K, V, positions):
        """Causal GQA.  q: [rows, H, D]; K, V: [KV, T, D]; row i sees keys 0..positions[i].

        Per query row and head h (KV head g = h // (H/KV)): scores z_t = (q . k_t) / sqrt(D)
        for t = 0..p, weights w = exp(z - max z), output sum_t w_t v_t / sum_t w_t.  Rows are
        taken in blocks as one score matrix per head; a key past a row's own position gets
        score -inf, so its weight is exactly zero and the row sees keys 0..p only.
        """
        H, KV, D = self.shape.n_heads, self.shape.n_kv_heads, self.shape.head_dim
        group = H // KV
        rows = q.shape[0]
        positions = np.asarray(positions)
        out = np.zeros((rows, H, D))
        scale = 1.0 / np.sqrt(D)
        blk = 256
        for r0 in range(0, rows, blk):
            r1 = min(rows, r0 + blk)
            pos = positions[r0:r1]
            n = int(pos.max()) + 1
            future = np.arange(n)[None, :] > pos[:, None]
            for h in range(H):
                g = h // group
                z = (q[r0:r1, h] @ K[g, :n].T) * scale
                z[future] = -np.inf
                w = np.exp(z - np.max(z, axis=1, keepdims=True))
                out[r0:r1, h] = (w @ V[g, :n]) / np.sum(w, axis=1, keepdims=True)
        return self._act(out)

    # ---- forward over new tokens of one sequence -------------------------------------

    def forward(self, seq: _Seq, ids, logits_rows: str = "last"):
        """Run ``ids`` (M new tokens) at positions seq.length .. seq.length+M-1.

        Appends to the sequence's KV cache and returns logits for the last row
        ([V]) or for every row ([M, V]).
        """
        sh = self.shape
        H, KV, D = sh.n_heads, sh.n_kv_heads, sh.head_dim
        ids = np.asarray(ids, dtype=np.int64).reshape(-1)
        if ids.size == 0:
            raise ValueError("empty token list")
        if ids.min() < 0 or ids.max() >= sh.vocab:
            raise ValueError("token id out of range")
        M = ids.size
        pos = np.arange(seq.length, seq.length + M)
        x = self.embed(ids)
        for li, L in enumerate(self.layers):
            h = self.rmsnorm(x, L["in_norm"])
            q = self.proj(L["q"], h).reshape(M, H, D)
            k = self.proj(L["k"], h).reshape(M, KV, D)
            v = self.proj(L["v"], h).reshape(M, KV, D)
            q = self.rmsnorm(q, L["q_norm"])
            k = self.rmsnorm(k, L["k_norm"])
            q = self.rope(q, pos)
            k = self.rope(k, pos)
            seq.k[li] = np.concatenate([seq.k[li], k.transpose(1, 0, 2)], axis=1)
            seq.v[li] = np.concatenate([seq.v[li], v.transpose(1, 0, 2)], axis=1)
            o = self.attention(q, seq.k[li], seq.v[li], pos).reshape(M, H * D)
            x = self._act(x + self.proj(L["o"], o))
            u = self.rmsnorm(x, L["post_norm"])
            gt = self.proj(L["gate"], u)
            up = self.proj(L["up"], u)
            a = self._act(gt / (1.0 + np.exp(-gt)) * up)
            x = self._act(x + self.proj(L["down"], a))
        seq.length += M
        xs = x if logits_rows == "all" else x[-1:]
        f = self.rmsnorm(xs, self.final_norm)
        logits = self._logit((f @ self.E_q.T) * self.E_s)
        return logits if logits_rows == "all" else logits[0]

    # ---- the greedy loop -------------------------------------------------------------

    def generate(self, prompt, n_new: int, teacher=None, keep_logits: bool = True):
        """Greedy decode of one sequence.

        Step 0 takes the arg-max of the prefill's last row; step k >= 1 feeds the
        previous step's token (or ``teacher[k-1]`` when teacher forcing) at
        position len(prompt) + k - 1.  Returns a dict with the generated ``ids``
        [n_new], per-step ``logits`` [n_new, V] (if kept) and ``margin`` [n_new]
        (top-1 minus top-2 logit).
        """
        if n_new < 1:
            raise ValueError("n_new must be >= 1")
        seq = self.new_sequence()
        ids, margins, all_logits = [], [], []
        logits = self.forward(seq, prompt)
        for k in range(n_new):
            if k > 0:
                feed = ids[k - 1] if teacher is None else int(teacher[k - 1])
                logits = self.forward(seq, [feed])
            t = greedy_argmax(logits)
            ids.append(t)
            top2 = np.partition(np.asarray(logits, dtype=np.float64), -2)[-2:]
            margins.append(float(top2[1] - top2[0]))
            if keep_logits:
                all_logits.append(np.asarray(logits))
        out = {"ids": np.array(ids, dtype=np.int32), "margin": np.array(margins)}
        if keep_logits:
            out["logits"] = np.stack(all_logits)
        return out
