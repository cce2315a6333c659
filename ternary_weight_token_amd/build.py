"""Compile the gfx950 library (libbitnet.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbitnet.so")

SOURCES = ["abi.cpp", "quant_act.hip", "pack.hip", "gemv.hip", "skinny.hip", "gemm.hip", "gemm_pipe.hip", "generic.hip", "bits.hip", "probe.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + (extra or []) + ["-I", os.path.join(ROOT, "include")] + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
