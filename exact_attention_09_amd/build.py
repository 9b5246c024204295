"""Build libfa355.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m exact_attention_09_amd.build`` (or ``build()`` from Python). The library is
written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa355.so")
OBJ = os.path.join(PKG, "_build")

SOURCES = ["fa355_api.hip", "fa_fwd_f16.hip", "fa_fwd_fp8.hip", "fa_bwd_f16.hip", "fa_decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU ops are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax reads and rescales them with VALU ops.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfa355.so. Returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
