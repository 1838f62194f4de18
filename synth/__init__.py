"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle side.

This module holds no arithmetic of the operator: it only draws inputs.
Values come from ``synth_gen.c`` (counter-based SplitMix64 draws,
Box-Muller normals), so a tensor is a pure function of
(seed, tensor id, flat index) and any row range can be regenerated alone.

Tensor ids: x / x1 = 0, x2 = 1, gamma = 2, beta = 3, smooth1 = 4,
smooth2 = 5, outlier columns = 6.

Workloads (shapes and distributions of the operator pages' use cases):

===========  ==========================================================
rmsnorm_dq   RmsNormDynamicQuant, x fp16 [64,1024] N(0,1), seed 0,
             gamma U(0.5,1.5), no beta, eps 1e-6, no smooth, int8 out
v2_square    AddRmsNormDynamicQuantV2 bf16 [4096,4096], seed 1, beta
             N(0,0.1), smooth1 U(0.5,2), mask [T,F], int8
v2_decode    bf16 [32,16384], seed 2, smooth1+2, mask [T,T], two int8
v2_outlier   bf16 [16384,8192], seed 3, 82 outlier columns x30 on x1
             and x2, smooth1+2, mask absent, two int8 outputs
v2_int4      fp16 [65536,5120], seed 4, smooth1 only, mask [T,F],
             y1 int4 (two codes per byte, low nibble first)
===========  ==========================================================
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gen.c")
_LIB = os.path.join(_HERE, "libsynth_gen.so")

DTYPES = {"bf16": 0, "fp16": 1}
NORMAL, UNIFORM = 0, 1
TID = {"x1": 0, "x2": 1, "gamma": 2, "beta": 3, "smooth1": 4, "smooth2": 5, "outlier": 6,
       "a_codes": 7, "a_scale": 8, "w_codes": 9, "w_scale": 10, "bias": 11,
       "lora_x": 12, "lora_y": 13, "lora_a": 14, "lora_b": 15, "lora_idx": 16}

_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
             "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_double, ctypes.c_double,
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_pick_columns.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.synth_pick_columns.restype = ctypes.c_int
        lib.synth_fill_int8.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_fill_int8.restype = ctypes.c_int
        lib.synth_fill_f32.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_double, ctypes.c_double,
            ctypes.c_int64, ctypes.c_void_p]
        lib.synth_fill_f32.restype = ctypes.c_int
        lib.synth_fill_i32.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p]
        lib.synth_fill_i32.restype = ctypes.c_int
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill(seed, tid, dist, p0, p1, dtype, rows, cols, row_offset=0, outlier=None,
         factor=1.0, out=None):
    """16-bit storage patterns of rows [row_offset, row_offset+rows) of a tensor."""
    if out is None:
        out = np.empty((rows, cols), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == rows * cols
    if outlier is not None:
        outlier = np.ascontiguousarray(outlier, dtype=np.uint8)
        assert outlier.size == cols
    rc = _load().synth_fill(
        int(seed), int(tid), int(dist), float(p0), float(p1), DTYPES[dtype], int(rows),
        int(cols), int(row_offset), None if outlier is None else outlier.ctypes.data,
        float(factor), _threads(), out.ctypes.data)
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return out


def pick_columns(seed, tid, n, k) -> np.ndarray:
    """0/1 flags of k distinct columns out of n (seeded partial Fisher-Yates)."""
    scratch = np.empty(n, dtype=np.int64)
    flags = np.empty(n, dtype=np.uint8)
    if _load().synth_pick_columns(int(seed), int(tid), int(n), int(k), scratch.ctypes.data,
                                  flags.ctypes.data) != 0:
        raise ValueError("bad column pick")
    return flags


@dataclass(frozen=True)
class Workload:
    name: str
    op: str  # "v2" (AddRmsNormDynamicQuantV2) or "rmsnorm" (RmsNormDynamicQuant)
    rows: int
    cols: int
    dtype: str
    seed: int
    mask: tuple | None
    has_beta: bool
    n_smooth: int
    y_types: tuple = ("int8", "int8")
    outlier_frac: float = 0.0
    outlier_factor: float = 30.0
    eps: float = 1e-6
    note: str = field(default="", compare=False)

    @property
    def n_outlier(self) -> int:
        return int(round(self.outlier_frac * self.cols))


WORKLOADS = {
    "rmsnorm_dq": Workload("rmsnorm_dq", "rmsnorm", 64, 1024, "fp16", 0, None, False, 0,
                           ("int8", "int8")),
    "v2_square": Workload("v2_square", "v2", 4096, 4096, "bf16", 1, (True, False), True, 1),
    "v2_decode": Workload("v2_decode", "v2", 32, 16384, "bf16", 2, (True, True), True, 2),
    "v2_outlier": Workload("v2_outlier", "v2", 16384, 8192, "bf16", 3, None, True, 2,
                           outlier_frac=0.01),
    "v2_int4": Workload("v2_int4", "v2", 65536, 5120, "fp16", 4, (True, False), True, 1,
                        ("int4", "int8")),
}


def params(w: Workload, cols=None, seed=None):
    """gamma, beta, smooth1, smooth2 ([cols] each, None when absent)."""
    cols = w.cols if cols is None else cols
    seed = w.seed if seed is None else seed
    g = fill(seed, TID["gamma"], UNIFORM, 0.5, 1.5, w.dtype, 1, cols)[0]
    b = fill(seed, TID["beta"], NORMAL, 0.0, 0.1, w.dtype, 1, cols)[0] if w.has_beta else None
    s1 = fill(seed, TID["smooth1"], UNIFORM, 0.5, 2.0, w.dtype, 1, cols)[0] \
        if w.n_smooth >= 1 else None
    s2 = fill(seed, TID["smooth2"], UNIFORM, 0.5, 2.0, w.dtype, 1, cols)[0] \
        if w.n_smooth >= 2 else None
    return g, b, s1, s2


def inputs(w: Workload, rows=None, row_offset=0, cols=None, seed=None):
    """x1 (and x2 for the V2 op) for a row range, N(0,1) with outlier columns."""
    rows = w.rows if rows is None else rows
    cols = w.cols if cols is None else cols
    seed = w.seed if seed is None else seed
    flags = None
    if w.outlier_frac > 0:
        flags = pick_columns(seed, TID["outlier"], cols, int(round(w.outlier_frac * cols)))
    x1 = fill(seed, TID["x1"], NORMAL, 0.0, 1.0, w.dtype, rows, cols, row_offset, flags,
              w.outlier_factor)
    x2 = None
    if w.op == "v2":
        x2 = fill(seed, TID["x2"], NORMAL, 0.0, 1.0, w.dtype, rows, cols, row_offset, flags,
                  w.outlier_factor)
    return x1, x2


def int8_codes(seed, tid, rows, cols, lo=-127, hi=127, row_offset=0) -> np.ndarray:
    """Uniform integers in [lo, hi], int8 [rows, cols]."""
    out = np.empty((rows, cols), dtype=np.int8)
    if _load().synth_fill_int8(int(seed), int(tid), int(lo), int(hi), int(rows), int(cols),
                               int(row_offset), out.ctypes.data) != 0:
        raise ValueError("synth_fill_int8 rejected its arguments")
    return out


def f32(seed, tid, dist, p0, p1, n) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if _load().synth_fill_f32(int(seed), int(tid), int(dist), float(p0), float(p1), int(n),
                              out.ctypes.data) != 0:
        raise ValueError("synth_fill_f32 rejected its arguments")
    return out


@dataclass(frozen=True)
class GemmWorkload:
    """INT8 GEMM consuming quantized activations: a [m, k] codes with one scale
    per row (as the operator's y1Out / scale1Out), w [n, k] codes with one
    scale per output column."""
    name: str
    m: int
    n: int
    k: int
    seed: int
    out_dtype: str = "bf16"
    has_bias: bool = False


GEMM_WORKLOADS = {
    # the headline activations (16384 rows of 8192) through an 8192 -> 8192 projection
    "w8a8_gemm": GemmWorkload("w8a8_gemm", 16384, 8192, 8192, 5),
}


def gemm_inputs(w: GemmWorkload, m=None, lo=-127, hi=127):
    """a codes, a_scale (U(0.01, 0.08): row max / 127 of activations of a few
    units), w codes, w_scale (U(1e-4, 1e-3)), bias (N(0, 0.1) or None)."""
    m = w.m if m is None else m
    a = int8_codes(w.seed, TID["a_codes"], m, w.k, lo, hi)
    sa = f32(w.seed, TID["a_scale"], UNIFORM, 0.01, 0.08, m)
    wq = int8_codes(w.seed, TID["w_codes"], w.n, w.k, lo, hi)
    sw = f32(w.seed, TID["w_scale"], UNIFORM, 1e-4, 1e-3, w.n)
    b = f32(w.seed, TID["bias"], NORMAL, 0.0, 0.1, w.n) if w.has_bias else None
    return a, sa, wq, sw, b


def int32s(seed, tid, lo, hi, n) -> np.ndarray:
    """Uniform integers in [lo, hi], int32 [n]."""
    out = np.empty(n, dtype=np.int32)
    if _load().synth_fill_i32(int(seed), int(tid), int(lo), int(hi), int(n),
                              out.ctypes.data) != 0:
        raise ValueError("synth_fill_i32 rejected its arguments")
    return out


@dataclass(frozen=True)
class LoraWorkload:
    """AddLora ("aclnnAddLora"): y [rows, h3] accumulates, in its columns
    [y_offset, y_offset + h2), scale * (x . A[g, layer]) . B[g, layer] for
    the adapter g = indices[row]; A is [w, l, h1, rank], B [w, l, rank, h2]."""
    name: str
    rows: int
    h1: int
    rank: int
    h2: int
    h3: int
    w: int
    l: int
    layer: int
    y_offset: int
    scale: float
    dtype: str
    seed: int
    idx_lo: int = 0          # indices uniform in [idx_lo, idx_hi]; outside [0, w) = no adapter
    idx_hi: int | None = None
    has_a: bool = True


LORA_WORKLOADS = {
    # a prefill batch of 4096 tokens over 8 adapters (all 32 layers' weights
    # resident), the k slice of a fused qkv output
    "lora_prefill": LoraWorkload("lora_prefill", 4096, 4096, 16, 4096, 12288, 8, 32, 7, 4096,
                                 0.5, "bf16", 6),
    # decode: 64 tokens, fp16
    "lora_decode": LoraWorkload("lora_decode", 64, 4096, 16, 4096, 12288, 8, 32, 7, 4096, 0.5,
                                "fp16", 7),
    # small case with ragged sizes and indices outside [0, w)
    "lora_small": LoraWorkload("lora_small", 300, 512, 16, 384, 1024, 5, 3, 2, 128, 0.25,
                               "bf16", 8, -1, 5),
}


def lora_inputs(wl: LoraWorkload, rows=None):
    """y, x (N(0, 1)), weight_a (N(0, 0.02), or None), weight_b (N(0, 0.02))
    as 16-bit storage patterns, and indices (int32)."""
    rows = wl.rows if rows is None else rows
    hi = wl.w - 1 if wl.idx_hi is None else wl.idx_hi
    y = fill(wl.seed, TID["lora_y"], NORMAL, 0.0, 1.0, wl.dtype, rows, wl.h3)
    x = fill(wl.seed, TID["lora_x"], NORMAL, 0.0, 1.0, wl.dtype, rows, wl.h1)
    wa = None
    if wl.has_a:
        wa = fill(wl.seed, TID["lora_a"], NORMAL, 0.0, 0.02, wl.dtype, wl.w * wl.l * wl.h1,
                  wl.rank).reshape(wl.w, wl.l, wl.h1, wl.rank)
    wb = fill(wl.seed, TID["lora_b"], NORMAL, 0.0, 0.02, wl.dtype, wl.w * wl.l * wl.rank,
              wl.h2).reshape(wl.w, wl.l, wl.rank, wl.h2)
    idx = int32s(wl.seed, TID["lora_idx"], wl.idx_lo, hi, rows)
    return y, x, wa, wb, idx
