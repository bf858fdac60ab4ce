"""Build libcc.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m ring_allreduce_reduction_02_amd.build_lib

Compiles every time it is called: each source file to an object in parallel
(in a temporary directory), then one link.  The library lands next to this
file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
import time
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcc.so")

SOURCES = [os.path.join(CSRC, f) for f in (
    "cc_kernels.hip", "cc_trees.hip", "cc_steps.hip", "cc_quant.hip", "cc_hier.hip", "cc_copy.hip", "cc_noalloc.hip",
    "cc_api.cpp", "cc_sched.cpp", "cc_alltoall.cpp", "cc_compress.cpp")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",              # no fused multiply-add: folds stay bit-exact
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unknown-pragmas",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    return r.stderr


def build(verbose: bool = True, extra_flags=(), out: str = LIB) -> str:
    """Compile and link; extra_flags go to every compile and the link."""
    t0 = time.time()
    tmpdir = tempfile.mkdtemp(prefix="cc_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in SOURCES]
        inc = ["-I", os.path.join(ROOT, "include")]
        cmds = [[hipcc(), *FLAGS, *extra_flags, *inc, "-c", "-o", o, s] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=max(1, min(len(cmds), os.cpu_count() or 1))) as ex:
            logs = list(ex.map(_run, cmds))
        tmp = out + ".tmp"
        logs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *extra_flags, "-o", tmp, *objs]))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        warn = [l for log in logs for l in log.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
        for l in warn[:20]:
            print(l)
        print(f"built {out} in {time.time() - t0:.1f}s")
    return out


if __name__ == "__main__":
    build()
