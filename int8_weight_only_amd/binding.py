"""ctypes binding of libqd.so (the C ABI in include/qd.h).

Argument marshalling only: PyTorch allocates the device buffers and supplies the
stream; every step of the forward pass runs in the library's HIP kernels.  The
binding raises if the built library is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqd.so")

QD_OK = 0
STATUS_CODES = {
    0: "ok",
    1: "unsupported_architecture",
    2: "invalid_arguments",
    3: "context_ceiling",
    4: "checkpoint_not_found",
    5: "buffer_too_small",
    6: "device_error",
    7: "cache_miss",
}
TENSORS = {"embed": 0, "q": 1, "k": 2, "v": 3, "o": 4, "gate": 5, "up": 6, "down": 7}
MAX_CONTEXT = 65536


class QdError(RuntimeError):
    """Error from the library; ``code`` is a stable string, ``status`` the C code."""

    def __init__(self, status: int, message: str):
        self.status = status
        self.code = STATUS_CODES.get(status, f"status_{status}")
        super().__init__(f"{self.code}: {message}")


class UnsupportedArchitectureError(QdError):
    pass


class ModelShapeC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("tie_word_embeddings", ctypes.c_int32),
                ("attention_bias", ctypes.c_int32)]


class LimitsC(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("max_prefill_tokens", ctypes.c_int32)]


class SizesC(ctypes.Structure):
    _fields_ = [("weight_bytes", ctypes.c_uint64), ("kv_bytes", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64), ("packed_model_bytes", ctypes.c_uint64)]


_P = ctypes.c_void_p


class LayerC(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("q", "k", "v", "o", "gate", "up", "down",
                                  "in_norm", "post_norm", "q_norm", "k_norm")]


class WeightsC(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("layers", ctypes.POINTER(LayerC))]


class BuffersC(ctypes.Structure):
    _fields_ = [("weights", _P), ("weight_bytes", ctypes.c_uint64), ("kv", _P),
                ("kv_bytes", ctypes.c_uint64), ("workspace", _P),
                ("workspace_bytes", ctypes.c_uint64)]


class StatsC(ctypes.Structure):
    _fields_ = [("prefill_us", ctypes.c_double), ("decode_us", ctypes.c_double),
                ("steps", ctypes.c_int32), ("n_prompt_tokens", ctypes.c_int32)]


EXPORTS = ("qd_last_error", "qd_check_shape", "qd_query_sizes", "qd_load_weights",
           "qd_export_quantized", "qd_prefill", "qd_decode_step", "qd_generate_greedy",
           "qd_free", "qd_profile_kernels", "qd_set_tuning", "qd_prefill_slots",
           "qd_decode_step_slots", "qd_sample", "qd_save_cache", "qd_load_cache",
           "qd_check_cache", "qd_sha256", "qd_run_op", "qd_sample_noalloc")
TUNING = {"attn_max_splits": 0, "attn_min_chunks": 1, "attn_waves": 2, "attn_merge_last": 3,
          "skinny_split": 6, "gemm_splits": 7, "attn_occupancy": 8, "skinny_norm": 9,
          "prefill_gemm": 10, "skinny_xstage": 11, "flash_rows": 12}
PROF_KERNELS = ("embed", "qkv", "attn", "o", "gateup", "down", "lmhead")
OPS = {"embed": 0, "qkv": 1, "o": 2, "gateup": 3, "down": 4, "lmhead": 5}

_lib = None


class SamplingC(ctypes.Structure):
    """qd_sampling: "Model-agnostic LLM inference", section "Sampling"."""
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("min_p", ctypes.c_float), ("top_p", ctypes.c_float),
                ("repeat_penalty", ctypes.c_float), ("presence_penalty", ctypes.c_float),
                ("frequency_penalty", ctypes.c_float)]


def load_library(path: str = LIB_PATH):
    """Load libqd.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m int8_weight_only_amd.build`")
    lib = ctypes.CDLL(path)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    lib.qd_last_error.restype = ctypes.c_char_p
    lib.qd_last_error.argtypes = []
    lib.qd_check_shape.restype = i32
    lib.qd_check_shape.argtypes = [ctypes.POINTER(ModelShapeC)]
    lib.qd_query_sizes.restype = i32
    lib.qd_query_sizes.argtypes = [ctypes.POINTER(ModelShapeC), ctypes.POINTER(LimitsC),
                                   ctypes.POINTER(SizesC)]
    lib.qd_load_weights.restype = i32
    lib.qd_load_weights.argtypes = [ctypes.POINTER(ModelShapeC), ctypes.POINTER(LimitsC),
                                    ctypes.POINTER(WeightsC), ctypes.POINTER(BuffersC), vp,
                                    ctypes.POINTER(vp)]
    lib.qd_export_quantized.restype = i32
    lib.qd_export_quantized.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.qd_prefill.restype = i32
    lib.qd_prefill.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    lib.qd_decode_step.restype = i32
    lib.qd_decode_step.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.qd_prefill_slots.restype = i32
    lib.qd_prefill_slots.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.qd_save_cache.restype = i32
    lib.qd_save_cache.argtypes = [vp, ctypes.c_char_p, vp, vp]
    lib.qd_load_cache.restype = i32
    lib.qd_load_cache.argtypes = [ctypes.POINTER(ModelShapeC), ctypes.POINTER(LimitsC),
                                  ctypes.c_char_p, vp, ctypes.POINTER(BuffersC), vp,
                                  ctypes.POINTER(vp)]
    lib.qd_check_cache.restype = i32
    lib.qd_check_cache.argtypes = [ctypes.POINTER(ModelShapeC), ctypes.c_char_p, vp]
    lib.qd_sha256.restype = i32
    lib.qd_sha256.argtypes = [vp, ctypes.c_uint64, vp]
    lib.qd_sample.restype = i32
    lib.qd_sample.argtypes = [vp, i32, vp, ctypes.POINTER(SamplingC), vp, vp, vp, vp]
    lib.qd_sample_noalloc.restype = i32
    lib.qd_sample_noalloc.argtypes = [vp, i32, vp, ctypes.POINTER(SamplingC), vp, vp, vp, vp]
    lib.qd_decode_step_slots.restype = i32
    lib.qd_decode_step_slots.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    lib.qd_generate_greedy.restype = i32
    lib.qd_generate_greedy.argtypes = [vp, i32, vp, vp, i32, i32, vp, vp,
                                       ctypes.POINTER(StatsC), vp]
    lib.qd_profile_kernels.restype = i32
    lib.qd_profile_kernels.argtypes = [vp, i32, i32, vp, vp]
    lib.qd_set_tuning.restype = i32
    lib.qd_set_tuning.argtypes = [vp, i32, i32]
    lib.qd_run_op.restype = i32
    lib.qd_run_op.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.qd_free.restype = None
    lib.qd_free.argtypes = [vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != QD_OK:
        msg = _lib.qd_last_error().decode()
        if status == 1:
            raise UnsupportedArchitectureError(status, msg)
        raise QdError(status, msg)


def shape_struct(shape) -> ModelShapeC:
    """C struct from any object with the config.json-style attributes."""
    return ModelShapeC(int(shape.hidden), int(shape.n_layers), int(shape.n_heads),
                       int(shape.n_kv_heads), int(shape.head_dim), int(shape.intermediate),
                       int(shape.vocab), float(shape.rms_eps), float(shape.rope_theta),
                       int(bool(getattr(shape, "tie_word_embeddings", True))),
                       int(bool(getattr(shape, "attention_bias", False))))


def _digest(d):
    d = bytes(d) if d is not None else b""
    if len(d) != 32:
        raise QdError(2, "source_digest must be 32 bytes")
    return ctypes.create_string_buffer(d, 32)


def sha256(data: bytes) -> bytes:
    """SHA-256 of ``data`` computed by the library."""
    load_library()
    buf = ctypes.create_string_buffer(bytes(data), max(1, len(data)))
    out = ctypes.create_string_buffer(32)
    _check(_lib.qd_sha256(buf, len(data), out))
    return out.raw


def check_cache(shape, path: str, source_digest: bytes):
    """The cache gate alone, on the host: raises QdError "cache_miss" naming the mismatch."""
    load_library()
    _check(_lib.qd_check_cache(ctypes.byref(shape_struct(shape)), str(path).encode(),
                               _digest(source_digest)))


def check_shape(shape):
    lib = load_library()
    s = shape_struct(shape)
    _check(lib.qd_check_shape(ctypes.byref(s)))


def query_sizes(shape, max_batch: int, max_ctx: int, max_prefill_tokens: int) -> dict:
    lib = load_library()
    s = shape_struct(shape)
    lim = LimitsC(max_batch, max_ctx, max_prefill_tokens)
    out = SizesC()
    _check(lib.qd_query_sizes(ctypes.byref(s), ctypes.byref(lim), ctypes.byref(out)))
    return {"weight_bytes": out.weight_bytes, "kv_bytes": out.kv_bytes,
            "workspace_bytes": out.workspace_bytes, "packed_model_bytes": out.packed_model_bytes}


def _stream_handle(stream=None) -> int:
    st = stream if stream is not None else torch.cuda.current_stream()
    return int(st.cuda_stream)


@dataclass
class GenerateResult:
    """Prompt + generated ids, as the pages' result record has them."""
    token_ids: list          # per sequence: prompt ids followed by generated ids
    n_prompt: list
    generated: np.ndarray    # [B, max_new_tokens] int32
    n_generated: np.ndarray  # [B]
    prefill_us: float
    decode_us: float
    steps: int
    prefill_tokens_per_sec: float
    decode_tokens_per_sec: float


class Model:
    """A loaded model: caller-owned device buffers plus the library handle."""

    def __init__(self, shape, weights: dict | None, max_batch: int = 1, max_ctx: int = 512,
                 max_prefill_tokens: int | None = None, device: str = "cuda:0",
                 cache_path: str | None = None, source_digest: bytes | None = None):
        """Quantizes ``weights`` (fp32 arrays) on the GPU, or, with ``weights=None``,
        restores the quantized cache at ``cache_path`` written for ``source_digest``
        (raises QdError code "cache_miss" when the cache fails its gate)."""
        lib = load_library()
        if not torch.cuda.is_available():
            raise QdError(6, "no GPU visible")
        self.shape = shape
        self.device = torch.device(device)
        self.max_batch, self.max_ctx = int(max_batch), int(max_ctx)
        self.max_prefill_tokens = int(max_prefill_tokens or max_batch * max_ctx)
        self._shape_c = shape_struct(shape)
        self._lim_c = LimitsC(self.max_batch, self.max_ctx, self.max_prefill_tokens)
        sizes = query_sizes(shape, self.max_batch, self.max_ctx, self.max_prefill_tokens)
        self.sizes = sizes
        with torch.cuda.device(self.device):
            self.wbuf = torch.empty(sizes["weight_bytes"], dtype=torch.uint8, device=self.device)
            self.kvbuf = torch.empty(sizes["kv_bytes"], dtype=torch.uint8, device=self.device)
            self.wsbuf = torch.empty(sizes["workspace_bytes"], dtype=torch.uint8, device=self.device)
            keep = []
            if weights is None:
                bufs = BuffersC(self.wbuf.data_ptr(), self.wbuf.numel(), self.kvbuf.data_ptr(),
                                self.kvbuf.numel(), self.wsbuf.data_ptr(), self.wsbuf.numel())
                handle = ctypes.c_void_p()
                st = torch.cuda.current_stream(self.device)
                dg = _digest(source_digest)
                _check(lib.qd_load_cache(ctypes.byref(self._shape_c), ctypes.byref(self._lim_c),
                                         str(cache_path).encode(), dg, ctypes.byref(bufs),
                                         _stream_handle(st), ctypes.byref(handle)))
                st.synchronize()
                self._h = handle
                return

            def dev(a):
                if a is None:
                    return None
                t = torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)
                keep.append(t)
                return t.data_ptr()

            layers = (LayerC * shape.n_layers)()
            for i, L in enumerate(weights["layers"]):
                layers[i] = LayerC(*[dev(L.get(k)) for k in
                                     ("q", "k", "v", "o", "gate", "up", "down",
                                      "in_norm", "post_norm", "q_norm", "k_norm")])
            wc = WeightsC(dev(weights.get("embed")), dev(weights.get("final_norm")), layers)
            bufs = BuffersC(self.wbuf.data_ptr(), self.wbuf.numel(), self.kvbuf.data_ptr(),
                            self.kvbuf.numel(), self.wsbuf.data_ptr(), self.wsbuf.numel())
            handle = ctypes.c_void_p()
            st = torch.cuda.current_stream(self.device)
            _check(lib.qd_load_weights(ctypes.byref(self._shape_c), ctypes.byref(self._lim_c),
                                       ctypes.byref(wc), ctypes.byref(bufs),
                                       _stream_handle(st), ctypes.byref(handle)))
            st.synchronize()
            del keep
        self._h = handle

    # ---- lifecycle ----------------------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            _lib.qd_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- calls ------------------------------------------------------------------------------
    def export_quantized(self, tensor: str, layer: int = 0):
        """int8 codes [rows, cols] and fp32 scales [rows] of one matrix, checkpoint layout."""
        s = self.shape
        qd_, kvd = s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim
        rc = {"embed": (s.vocab, s.hidden), "q": (qd_, s.hidden), "k": (kvd, s.hidden),
              "v": (kvd, s.hidden), "o": (s.hidden, qd_), "gate": (s.intermediate, s.hidden),
              "up": (s.intermediate, s.hidden), "down": (s.hidden, s.intermediate)}[tensor]
        q = np.empty(rc, dtype=np.int8)
        sc = np.empty(rc[0], dtype=np.float32)
        _check(_lib.qd_export_quantized(self._h, TENSORS[tensor], layer, q.ctypes.data,
                                        sc.ctypes.data, _stream_handle()))
        return q, sc

    def prefill(self, prompts, logits: bool = False, slots=None):
        """Prefill prompts into slots 0..n-1 (or into the KV slots ``slots``, one per prompt).
        Returns (next_ids [n] int32 cuda, logits [n, V] or None)."""
        prompts = [np.asarray(p, dtype=np.int32).reshape(-1) for p in prompts]
        lens = np.array([p.size for p in prompts], dtype=np.int32)
        flat = np.concatenate(prompts) if prompts else np.zeros(0, np.int32)
        ids_dev = torch.from_numpy(flat).to(self.device)
        nxt = torch.empty(len(prompts), dtype=torch.int32, device=self.device)
        lg = torch.empty((len(prompts), self.shape.vocab), dtype=torch.float32,
                         device=self.device) if logits else None
        lg_ptr = lg.data_ptr() if lg is not None else None
        if slots is None:
            _check(_lib.qd_prefill(self._h, len(prompts), ids_dev.data_ptr(), flat.ctypes.data,
                                   lens.ctypes.data, lg_ptr, nxt.data_ptr(), _stream_handle()))
        else:
            sl = np.ascontiguousarray(slots, dtype=np.int32).reshape(-1)
            _check(_lib.qd_prefill_slots(self._h, len(prompts), sl.ctypes.data, ids_dev.data_ptr(),
                                         flat.ctypes.data, lens.ctypes.data, lg_ptr,
                                         nxt.data_ptr(), _stream_handle()))
        return nxt, lg

    def decode_step(self, in_ids, logits: bool = False, slots=None):
        """One step for slots 0..B-1 (or the KV slots ``slots``, row b = slots[b]) fed
        ``in_ids`` (int32 cuda tensor [B])."""
        in_ids = torch.as_tensor(in_ids, dtype=torch.int32).to(self.device).contiguous()
        B = in_ids.numel()
        nxt = torch.empty(B, dtype=torch.int32, device=self.device)
        lg = torch.empty((B, self.shape.vocab), dtype=torch.float32,
                         device=self.device) if logits else None
        lg_ptr = lg.data_ptr() if lg is not None else None
        if slots is None:
            _check(_lib.qd_decode_step(self._h, B, in_ids.data_ptr(), lg_ptr, nxt.data_ptr(),
                                       _stream_handle()))
        else:
            sl = np.ascontiguousarray(slots, dtype=np.int32).reshape(-1)
            if sl.size != B:
                raise QdError(2, f"{sl.size} slots for {B} ids")
            _check(_lib.qd_decode_step_slots(self._h, B, sl.ctypes.data, in_ids.data_ptr(), lg_ptr,
                                             nxt.data_ptr(), _stream_handle()))
        return nxt, lg

    def save_cache(self, path: str, source_digest: bytes):
        """Writes the quantized weights to ``path`` (the quantized load cache)."""
        _check(_lib.qd_save_cache(self._h, str(path).encode(), _digest(source_digest),
                                  _stream_handle()))

    def sample(self, logits, seeds, slots=None, temperature=1.0, top_k=40, min_p=0.0,
               top_p=1.0, repeat_penalty=1.0, presence_penalty=0.0, frequency_penalty=0.0,
               noalloc=False):
        """Draws one id per row of ``logits`` (fp32 cuda [B, V]) for slots 0..B-1 (or
        ``slots``) with per-row ``seeds``; returns int32 cuda [B].  noalloc=True calls
        qd_sample_noalloc (the library's fixed scratch; at most 16 rows, rows x V <= 2^21)."""
        logits = logits.contiguous()
        B = logits.shape[0]
        sd = np.ascontiguousarray(seeds, dtype=np.uint64).reshape(-1)
        if sd.size != B:
            raise QdError(2, f"{sd.size} seeds for {B} rows")
        sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int32).reshape(-1)
        if sl is not None and sl.size != B:
            raise QdError(2, f"{sl.size} slots for {B} rows")
        prm = SamplingC(temperature, top_k, min_p, top_p, repeat_penalty, presence_penalty,
                        frequency_penalty)
        nxt = torch.empty(B, dtype=torch.int32, device=self.device)
        fn = _lib.qd_sample_noalloc if noalloc else _lib.qd_sample
        _check(fn(self._h, B, sl.ctypes.data if sl is not None else None,
                  ctypes.byref(prm), sd.ctypes.data, logits.data_ptr(),
                  nxt.data_ptr(), _stream_handle()))
        return nxt

    def set_tuning(self, **knobs):
        """Launch-policy knobs, e.g. attn_max_splits=8 (performance only)."""
        for k, v in knobs.items():
            _check(_lib.qd_set_tuning(self._h, TUNING[k], int(v)))

    def profile_kernels(self, B: int, iters: int = 50) -> dict:
        """Mean microseconds per launch of each decode-step kernel class (HIP events)."""
        us = np.zeros(len(PROF_KERNELS), dtype=np.float32)
        _check(_lib.qd_profile_kernels(self._h, int(B), int(iters), us.ctypes.data,
                                       _stream_handle()))
        return dict(zip(PROF_KERNELS, map(float, us)))

    def run_op(self, op: str, x, resid=None, layer: int = 0):
        """One decode-step kernel class on caller inputs (qd_run_op): ``x`` is int32 ids [B]
        for "embed", else a bf16 cuda tensor [B, K]; ``resid`` bf16 [B, hidden] for "o" and
        "down".  Returns the output tensor (and, for "lmhead", (logits, ids))."""
        s = self.shape
        x = x.contiguous()
        B = x.shape[0]
        width = {"embed": s.hidden, "qkv": (s.n_heads + 2 * s.n_kv_heads) * s.head_dim,
                 "o": s.hidden, "gateup": s.intermediate, "down": s.hidden, "lmhead": s.vocab}[op]
        dt = torch.float32 if op == "lmhead" else torch.bfloat16
        out = torch.empty((B, width), dtype=dt, device=self.device)
        ids = torch.empty(B, dtype=torch.int32, device=self.device) if op == "lmhead" else None
        r = resid.contiguous() if resid is not None else None
        _check(_lib.qd_run_op(self._h, OPS[op], int(layer), int(B), x.data_ptr(),
                              r.data_ptr() if r is not None else None, out.data_ptr(),
                              ids.data_ptr() if ids is not None else None, _stream_handle()))
        return (out, ids) if op == "lmhead" else out

    def generate_greedy(self, prompts, max_new_tokens: int, eos_id: int = -1) -> GenerateResult:
        """Prefill + (max_new_tokens - 1) decode steps, greedy, in one library call."""
        prompts = [np.asarray(p, dtype=np.int32).reshape(-1) for p in prompts]
        B = len(prompts)
        lens = np.array([p.size for p in prompts], dtype=np.int32)
        flat = np.ascontiguousarray(np.concatenate(prompts)) if B else np.zeros(0, np.int32)
        out = np.zeros((max(B, 1), max(int(max_new_tokens), 1)), dtype=np.int32)
        n_out = np.zeros(max(B, 1), dtype=np.int32)
        st = StatsC()
        _check(_lib.qd_generate_greedy(self._h, B, flat.ctypes.data, lens.ctypes.data,
                                       int(max_new_tokens), int(eos_id), out.ctypes.data,
                                       n_out.ctypes.data, ctypes.byref(st), _stream_handle()))
        toks = [list(map(int, prompts[b])) + list(map(int, out[b, :n_out[b]])) for b in range(B)]
        dec_tok = B * st.steps
        return GenerateResult(
            token_ids=toks, n_prompt=[int(x) for x in lens], generated=out, n_generated=n_out,
            prefill_us=st.prefill_us, decode_us=st.decode_us, steps=st.steps,
            prefill_tokens_per_sec=(lens.sum() / (st.prefill_us * 1e-6)) if st.prefill_us > 0 else 0.0,
            decode_tokens_per_sec=(dec_tok / (st.decode_us * 1e-6)) if st.decode_us > 0 else 0.0)
