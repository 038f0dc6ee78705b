"""Build the HIP library ``libsdm.so`` in-tree for gfx950.

    python -m sparse_memory_linear_pkm_amd.build

Every translation unit under ``csrc/`` is compiled with hipcc for gfx950
only, then linked into ``sparse_memory_linear_pkm_amd/libsdm.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsdm.so")
# measurement-only kernels (bench.py), kept out of the SDM library
BENCH_CSRC = os.path.join(HERE, "bench_csrc")
BENCH_LIB = os.path.join(HERE, "libsdm_bench.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed fp32 ops are switched off for all device code.  No floating-point
# contraction: every fused multiply-add is written out (__builtin_fmaf), so
# each result has one fixed rounding sequence wherever it is computed (the
# decode step reproduces the prefill scan bit for bit).
CFLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    bsrcs = sorted(glob.glob(os.path.join(BENCH_CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(bsrcs))) as ex:
        objs = list(ex.map(_compile, srcs + bsrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
