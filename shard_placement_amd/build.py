"""Build libtide.so in-tree with hipcc for gfx950.

All device code is compiled for gfx950 only, at -O3, without fast-math or
denormal flushing (the reduction must be IEEE binary32 with subnormals), and
with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtide.so")
SOURCES = ["plan.cpp", "rs.hip", "ag.hip", "dma.cpp", "pipeline.cpp"]
LIBS = ["-L/opt/rocm/lib", "-lhsa-runtime64"]  # ROCr, for the copy engines
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + LIBS + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
