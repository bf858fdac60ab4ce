"""Build libcc.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m ring_allreduce_reduction_02_amd.build_lib

Compiles every time it is called.  The library lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcc.so")

SOURCES = [os.path.join(CSRC, "cc_kernels.hip"), os.path.join(CSRC, "cc_api.cpp"), os.path.join(CSRC, "cc_sched.cpp"),
           os.path.join(CSRC, "cc_alltoall.cpp"), os.path.join(CSRC, "cc_compress.cpp"),
           os.path.join(CSRC, "cc_noalloc.hip")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",              # no fused multiply-add: folds stay bit-exact
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unknown-pragmas",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(tmp, LIB)
    if verbose:
        warn = [l for l in r.stderr.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
        for l in warn[:20]:
            print(l)
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build()
