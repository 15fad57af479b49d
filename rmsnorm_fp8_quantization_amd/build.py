"""Build the gfx950 library ``libnormfp8.so`` in-tree with hipcc.

Usage: ``python -m rmsnorm_fp8_quantization_amd.build`` (or ``build()`` from Python).
Every translation unit is compiled ahead of time for gfx950 only; objects go to
``_build/`` next to this file and the shared library lands in the package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnormfp8.so")
SOURCES = ["api.cpp", "fwd_row.hip", "fwd_band.hip", "fwd_col.hip", "bwd.hip", "gen.hip", "noalloc.hip", "fwd_split.hip", "fwd_colx.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
            # a local that shadows another (e.g. an array hiding a bool guard) is an error
            "-Wshadow", "-Werror=shadow", "-Werror=pointer-bool-conversion",
            # never emit packed fp32 VALU ops (v_pk_*_f32)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, jobs: int = 0) -> str:
    """Compile every source and link ``libnormfp8.so``; returns the library path."""
    t0 = time.time()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
