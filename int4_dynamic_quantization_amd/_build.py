"""Build libaddrmsnorm_dq.so in-tree with hipcc for gfx950.

Each source compiles to its own object in parallel, then one link step.
Usage: python -m int4_dynamic_quantization_amd._build
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
LIB = os.path.join(PKG, "libaddrmsnorm_dq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["adq_api.cpp", "adq_row_bf16.hip", "adq_row_f16.hip", "adq_generic.hip",
           "adq_split.hip", "adq_gemm.hip", "adq_lora.hip"]
COMMON = ["-O3", "-fPIC", "-std=c++20", "-Wall", "-Wextra", "-Wno-unused-parameter",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only, with packed-fp32 (v_pk_*_f32) generation
# turned off; the kernels are written with scalar fp32 arithmetic.
# Code object v5 loads under every HIP runtime this library may bind to.
DEVICE = [f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", "-c", path, "-o", obj] + COMMON + DEVICE
    else:
        cmd = [HIPCC, "-c", path, "-o", obj] + COMMON + ["-D__HIP_PLATFORM_AMD__"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    missing = [s for s in SOURCES if not os.path.exists(os.path.join(CSRC, s))]
    if missing:
        raise FileNotFoundError(f"missing sources in {CSRC}: {', '.join(missing)}")
    srcs = list(SOURCES)
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
