"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/host_sanitize/build.py compiles qd_api.hip for the host only and qd_cache.cpp with both
sanitizers (no GPU code is built with them) and links them with a harness that drives the C
ABI through every path that needs no GPU: the architecture gates and named errors
("Model-agnostic LLM inference", sections "Supported models" and "Errors"), buffer sizing,
SHA-256 against the example digests of FIPS 180-4, and the quantized load cache's gate
("The quantized load cache") on well-formed, truncated, extended and damaged files.  A
sanitizer report aborts the harness, so exit status 0 with "ok" means none was made.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(not os.path.exists("/opt/rocm/llvm/bin/clang++"), reason="no ROCm clang++")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    sys.path.insert(0, os.path.join(HERE, "host_sanitize"))
    from build import build
    exe = build(str(tmp_path / "build"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
