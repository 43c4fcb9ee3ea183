"""Builds the HIP library libmoe_latent.so in-tree for gfx950 with hipcc.

Always recompiles every source (no stale objects: the header is part of every
translation unit). Usage: python -m latent_moe_expert_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_latent.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for all device code.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]

SOURCES = ["api.cpp", "dense.hip", "dense_gemv.hip", "gemm.hip", "router.hip", "align.hip", "mxfp4_small.hip",
           "mxfp4_mfma.hip", "quant.hip", "combine.hip", "qb.hip", "stream.hip"]


def _compile(src: str, build_dir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, out: str = LIB, build_dir: str = BUILD, extra_flags: tuple = ()) -> str:
    """Compile every source and link `out`. extra_flags go to every compile and to the link
    (the CPU tests build a copy whose host code carries the address and undefined-behaviour
    sanitizers this way)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, tuple(extra_flags)), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra_flags, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
