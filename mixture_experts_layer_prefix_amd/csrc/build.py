"""Build libmoe.so (all HIP sources of the package) for gfx950 with hipcc.

Usage: python -m mixture_experts_layer_prefix_amd.csrc.build
Writes mixture_experts_layer_prefix_amd/libmoe.so next to the package.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
OUT = os.path.join(PKG, "libmoe.so")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "*.hip")))


def build(verbose: bool = True) -> str:
    srcs = sources()
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(os.path.dirname(PKG), "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
