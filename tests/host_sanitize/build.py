"""Builds the host-code sanitizer harness: the library's host side (qd_api.hip compiled for
the host only, qd_cache.cpp) with AddressSanitizer and UndefinedBehaviorSanitizer, the
device-side launchers replaced by stand-ins (stubs.hip), and harness.cpp.  No GPU code is
built with a sanitizer: every hipcc line compiles host code only and passes each
-fsanitize= behind -Xarch_host; the C++-only files and the link use clang++.

Usage: python tests/host_sanitize/build.py OUT_DIR  (prints the harness path)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "int8_weight_only_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", CSRC]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
CPP_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    o = lambda n: os.path.join(out_dir, n)
    steps = [
        [HIPCC, *COMMON, "--cuda-host-only", *HOST_SAN, "-c", os.path.join(CSRC, "qd_api.hip"), "-o", o("api.o")],
        [HIPCC, *COMMON, "--cuda-host-only", *HOST_SAN, "-c", os.path.join(HERE, "stubs.hip"), "-o", o("stubs.o")],
        [CLANG, *COMMON, *CPP_SAN, "-c", os.path.join(CSRC, "qd_cache.cpp"), "-o", o("cache.o")],
        [CLANG, *COMMON, *CPP_SAN, "-c", os.path.join(HERE, "harness.cpp"), "-o", o("harness.o")],
        [CLANG, *CPP_SAN, o("api.o"), o("stubs.o"), o("cache.o"), o("harness.o"),
         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-o", o("harness")],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")
    return o("harness")


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "host_sanitize")))
