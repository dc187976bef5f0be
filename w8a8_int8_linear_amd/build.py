"""Build libsmoothquant.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

    python w8a8_int8_linear_amd/build.py         # compiles every source, links the library

(Run it as a file: importing the package first would load the library being built.)
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsmoothquant.so")
ARCH = os.environ.get("SQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["sq_validate.cpp", "sq_api.cpp", "k_rows.hip", "k_rows_tensor.hip", "k_rows_step.hip", "k_rows_fp8.hip",
           "k_rows_fp8_step.hip", "k_gemm.hip", "k_llm_int8.hip", "sq_noalloc.hip"]

# Numerics: no contraction of separate roundings, IEEE fp32 divide/sqrt, binary32
# denormals kept. Packed fp32 instructions are disabled for all device code.
COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs where they fit: the AGPR form rotates registers
    # through copies inside the GEMM main loop.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsmoothquant.so")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if noise:
            sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
