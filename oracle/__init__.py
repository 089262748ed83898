"""CPU oracle for the int8 weight-only Qwen3 decoder step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the product library or its binding.
"""
from .qwen3_int8 import (bf16, quantize_rows, quantize_model, Oracle, greedy_argmax,
                         packed_weight_bytes)

__all__ = ["bf16", "quantize_rows", "quantize_model", "Oracle", "greedy_argmax",
           "packed_weight_bytes"]
