"""Builds the tests' own GPU helper (tests/silu_check.hip) into
tests/_build/libsilu_check.so, with the library's compiler flags, so that the
GPU test compares the library's device SiLU exactly as the kernels compile
it.  Called by __graft_entry__.build(); test infrastructure."""
from __future__ import annotations

import os
import subprocess

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
OUT = os.path.join(TESTS, "_build", "libsilu_check.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "w8a8_quantized_moe_amd", "csrc"),
           "-I", TESTS, "-x", "hip", os.path.join(TESTS, "silu_check.hip"), "-o", OUT + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for silu_check.hip:\n{r.stderr}")
    os.replace(OUT + ".tmp", OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
