"""Build the C++ client of the kvq C ABI (tests/c_client/kvq_c_client) against
the in-tree libkvq.so and the oracle's liborc.so.  The client is host code
only, so g++ with the HIP runtime headers builds it; both libraries must be
built first.

    python tests/c_client/build_client.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "kvq_c_client.cpp")
BIN = os.path.join(HERE, "kvq_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = BIN + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", tmp,
           "-L", os.path.join(ROOT, "quantized_kv_cache_fp8_amd"), "-lkvq",
           "-L", os.path.join(ROOT, "oracle"), "-lorc",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../quantized_kv_cache_fp8_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for {SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
    sys.exit(0)
