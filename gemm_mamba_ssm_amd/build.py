"""Builds libw8a16.so (gfx950 only) in-tree with hipcc.

    python -m gemm_mamba_ssm_amd.build

Each HIP source compiles to an object in parallel, then one shared library is
linked. Packed FP32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw8a16.so")
ARCH = "gfx950"

SOURCES = ["w8a16_common.cpp", "w8a16_gemv.hip", "w8a16_gemm.hip", "w8a16_gemm_wide.hip", "w8a16_skinny.hip",
           "w8a16_mid.hip", "w8a16_dequant.hip", "w8a16_norm.hip", "w8a16_mamba2.hip", "w8a16_read.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7.x with gfx950 support is required)")


def _compile(hipcc: str, src: str, extra: list[str]) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc, *HIPCC_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra_flags: list[str] | None = None, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libw8a16.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra_flags or [])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, extra), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
