"""Build libpql.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m precision_quantized_linear_amd.build

Each source compiles to an object in ``_build/`` (in parallel), then links
into ``precision_quantized_linear_amd/libpql.so``.  Packed-fp32 VALU ops are
disabled (``-packed-fp32-ops``) for every device compile.
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
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpql.so")
SOURCES = ("abi.cpp", "quant.hip", "layout.hip", "gemm.hip", "gemm32.hip", "gemm_block.hip", "gemm_block256.hip", "gemm_w4a16.hip", "gemm_dual.hip", "qlinear_small.hip",
           "gemm_w4a16_mm.hip")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpql")
    return path


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-file code-generation options.  The block-128 GEMM promotes every matrix-core
# partial product with VALU FMAs; taking the MFMA results in VGPRs (instead of
# AGPRs) spares one v_accvgpr_read per element.
EXTRA_FLAGS = {"gemm_block.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "gemm_block256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
