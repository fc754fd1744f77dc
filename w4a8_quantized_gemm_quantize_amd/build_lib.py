"""Compile libw4a8.so (the HIP/gfx950 library behind include/w4a8.h) in-tree.

Flags that matter for results:
  -ffp-contract=off   no fused multiply-add is formed from separate * and +,
                      so every binary32 step rounds exactly once as written;
  (default)           binary32 division is correctly rounded in HIP;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libw4a8.so")
SOURCES = ["abi.hip", "quantize.hip", "pack.hip", "gemm_w4.hip", "gemm_lqq.hip", "gemm_w8.hip", "equarx.hip", "gemm_blockact.hip", "probe.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(out: str = LIB, extra=()) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", INCLUDE, "-I", CSRC, *extra, "-o", out,
            *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    cmd = command(LIB + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
