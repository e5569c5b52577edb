"""Build libmoe.so (all HIP sources of the package) for gfx950 with hipcc.

Usage: python -m mixture_experts_layer_prefix_amd.csrc.build
Writes mixture_experts_layer_prefix_amd/libmoe.so next to the package.

Each translation unit is compiled to an object of its own (in parallel, into
_build/ at the repository root), then the objects are linked into the shared
library.  Device code never crosses translation units (every device helper
is an inline function of a header), so no relocatable device code is needed.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libmoe.so")
OBJ_DIR = os.path.join(ROOT, "_build")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "*.hip")))


def _jobs() -> int:
    n = os.cpu_count() or 8
    return max(1, min(16, n))


def build(verbose: bool = True) -> str:
    srcs = sources()
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
        cmd = [HIPCC, *FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, r

    with ThreadPoolExecutor(_jobs()) as ex:
        results = list(ex.map(compile_one, srcs))
    failed = [(s, r) for s, _, r in results if r.returncode != 0]
    for s, _, r in results:
        # the host pass does not know the packed-fp32 feature: that warning is harmless
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip():
            print(err, file=sys.stderr, flush=True)
    if failed:
        raise subprocess.CalledProcessError(failed[0][1].returncode, f"hipcc -c {failed[0][0]}")
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _ in results],
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
