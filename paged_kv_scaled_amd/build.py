"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_scaled_amd.build            # compile + link
Objects go to paged_kv_scaled_amd/_build/ (git-ignored); the shared library is
paged_kv_scaled_amd/libpkv.so, next to the binding that loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
# the benchmark's achievable-ceiling kernels (a streaming read, an MFMA-only loop): a
# library of their own, loaded by bench.py only
LIB_CEILINGS = os.path.join(PKG, "libpkv_ceilings.so")
CEILING_SOURCES = ["ceilings.hip"]

SOURCES = ["api.cpp", "scatter.hip", "decode.hip", "prefill_valu.hip", "prefill_mfma.hip",
           "smallseq.hip", "checks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=fast", "-Werror=array-bounds",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-file code-generation options.  The MFMA prefill kernel keeps its accumulators in
# VGPRs (VGPR-form MFMA): with the default AGPR form the compiler copies the output
# accumulator between register files on every key tile.  It also runs with the IEEE mode
# bit off and NaN-free inputs assumed: in IEEE mode every fmax operand that comes out of an
# MFMA is first canonicalised (one extra VALU op per score), and NaN keys or queries give
# undefined results either way.
_MFMA_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"]
# The decode kernels' matrix-core core keeps its accumulators in VGPRs for the same reason,
# but stays in IEEE mode: decode results with NaN inputs are defined (NaN rows).
EXTRA = {"prefill_mfma.hip": _MFMA_FLAGS,
         "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], LIB_CEILINGS)
    if verbose:
        print(f"built {LIB} and {LIB_CEILINGS}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
