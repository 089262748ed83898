"""int8 weight-only Qwen3-family decoding on AMD MI355X (gfx950).

The product is the C-ABI library ``libqd.so`` (include/qd.h) with hand-written HIP
kernels; this package is its thin Python binding.
"""
from .binding import (Model, GenerateResult, QdError, UnsupportedArchitectureError,
                      check_shape, query_sizes, load_library, EXPORTS, LIB_PATH, MAX_CONTEXT,
                      sha256, check_cache)

__all__ = ["Model", "GenerateResult", "QdError", "UnsupportedArchitectureError", "check_shape",
           "query_sizes", "load_library", "EXPORTS", "LIB_PATH", "MAX_CONTEXT", "sha256", "check_cache"]
