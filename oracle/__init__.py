"""CPU oracle for fused (Add)RmsNorm + per-row symmetric dynamic quantization.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import this package.  The product
library never loads it, and it shares no code with the GPU path: the
arithmetic lives in ``adq_oracle.c`` (plain C, double precision, one row
at a time); this module only marshals numpy arrays into it.

Formulas followed: "aclnnAddRmsNormDynamicQuantV2", Formula and
Constraints sections; "aclnnRmsNormDynamicQuant", formula section
(计算公式); "aclnnAddLora", Formulas.  See the header of ``adq_oracle.c`` for every reading taken
where the pages are silent.

Pins (what checks this oracle against something other than itself) are in
``tests/test_oracle_pins.py``: hand-worked rows from the formulas stored in
``tests/golden/``, closed forms, exact-rational brute force and invariants.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "adq_oracle.c")
_LIB = os.path.join(_HERE, "libadq_oracle.so")

DTYPES = {"bf16": 0, "fp16": 1}
QMAX = {"int8": 127, "int4": 7}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libadq_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_storage_value.argtypes = [ctypes.c_uint16, ci]
    lib.oracle_storage_value.restype = ctypes.c_double
    lib.oracle_round_to_storage.argtypes = [ctypes.c_double, ci]
    lib.oracle_round_to_storage.restype = ctypes.c_uint16
    lib.oracle_v2_outputs.argtypes = [p, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci)]
    lib.oracle_v2_outputs.restype = ci
    lib.oracle_add_rms_norm_dq.argtypes = [
        i64, i64, ci, p, p, p, p, p, p, ctypes.c_double, ci, ci,
        p, p, p, p, p, p, p, p]
    lib.oracle_add_rms_norm_dq.restype = ci
    lib.oracle_pack_int4.argtypes = [i64, i64, p, p]
    lib.oracle_pack_int4.restype = ci
    lib.oracle_w8a8_gemm_at.argtypes = [i64, p, p, i64, p, p, p, p, p, p, p]
    lib.oracle_w8a8_gemm_at.restype = ci
    lib.oracle_add_lora.argtypes = [i64, i64, i64, i64, i64, i64, i64, ci, p, p, p, p, p, i64,
                                    ctypes.c_double, i64, i64, p, p, p, p]
    lib.oracle_add_lora.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Route every oracle call to another build of adq_oracle.c (used by the
    tests that plant mistakes in a copy of the oracle and check that the pins
    catch them)."""
    global _lib
    saved = _lib
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(a, n=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if n is not None and a.size != n:
        raise ValueError(f"parameter vector has {a.size} entries, expected {n}")
    return a


def storage_value(bits, dtype: str) -> float:
    """Exact value of one 16-bit storage pattern."""
    return _load().oracle_storage_value(int(bits), DTYPES[dtype])


def round_to_storage(value: float, dtype: str) -> int:
    """Nearest storage value (ties to even) of a double, as its bit pattern."""
    return int(_load().oracle_round_to_storage(float(value), DTYPES[dtype]))


def v2_outputs(mask, has_s1: bool, has_s2: bool):
    """(valid, y1_active, y2_active) of an AddRmsNormDynamicQuantV2 call."""
    lib = _load()
    a1, a2 = ctypes.c_int(0), ctypes.c_int(0)
    m = None
    if mask is not None:
        m = (ctypes.c_int * 2)(int(bool(mask[0])), int(bool(mask[1])))
    ok = lib.oracle_v2_outputs(m, int(bool(has_s1)), int(bool(has_s2)),
                               ctypes.byref(a1), ctypes.byref(a2))
    return bool(ok), bool(a1.value), bool(a2.value)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    rows, n = codes.shape
    out = np.empty((rows, n // 2), dtype=np.uint8)
    if _load().oracle_pack_int4(rows, n, _ptr(codes), _ptr(out)) != 0:
        raise ValueError("INT4 packing needs an even last dimension")
    return out


def _run(x1, x2, gamma, beta, s1, s2, eps, q1, q2, dtype, want_xout, want_pre):
    x1 = np.ascontiguousarray(x1, dtype=np.uint16)
    rows, n = x1.shape
    x2 = None if x2 is None else np.ascontiguousarray(x2, dtype=np.uint16)
    if x2 is not None and x2.shape != x1.shape:
        raise ValueError("x1 and x2 differ in shape")
    gamma, beta, s1, s2 = (_u16(t, n) for t in (gamma, beta, s1, s2))
    out = {}
    x_out = np.empty((rows, n), np.uint16) if want_xout else None
    c = [np.zeros((rows, n), np.int8) if q else None for q in (q1, q2)]
    sc = [np.zeros(rows, np.float32) if q else None for q in (q1, q2)]
    pr = [np.zeros((rows, n), np.float64) if (q and want_pre) else None for q in (q1, q2)]
    work = np.empty(2 * n, np.float64)
    rc = _load().oracle_add_rms_norm_dq(
        rows, n, DTYPES[dtype], _ptr(x1), _ptr(x2), _ptr(gamma), _ptr(beta), _ptr(s1),
        _ptr(s2), float(eps), int(q1), int(q2), _ptr(x_out), _ptr(c[0]), _ptr(c[1]),
        _ptr(sc[0]), _ptr(sc[1]), _ptr(pr[0]), _ptr(pr[1]), _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if want_xout:
        out["x_out"] = x_out
    for k in range(2):
        if (q1, q2)[k]:
            out[f"code{k + 1}"] = c[k]
            out[f"scale{k + 1}"] = sc[k]
            if want_pre:
                out[f"pre{k + 1}"] = pr[k]
    return out


def add_rms_norm_dq_v2(x1, x2, gamma, beta=None, smooth1=None, smooth2=None, eps=1e-6,
                       mask=None, y1_type="int8", y2_type="int8", dtype="bf16",
                       want_pre=True):
    """AddRmsNormDynamicQuantV2 on host arrays of 16-bit storage patterns.

    Returns a dict with ``x_out`` and, for each produced output k,
    ``code{k}`` (int8 codes, INT4 unpacked), ``scale{k}`` (float32),
    ``pre{k}`` (double input/scale before rounding) and, for INT4,
    ``packed{k}`` (two codes per byte, low nibble first).  Raises
    ValueError for a call the Constraints section forbids.
    """
    ok, a1, a2 = v2_outputs(mask, smooth1 is not None, smooth2 is not None)
    if not ok:
        raise ValueError("outputMask / smooth-scale combination not allowed")
    q1 = QMAX[y1_type] if a1 else 0
    q2 = QMAX[y2_type] if a2 else 0
    out = _run(x1, x2, gamma, beta, smooth1, smooth2, eps, q1, q2, dtype, True, want_pre)
    for k, (act, t) in enumerate(((a1, y1_type), (a2, y2_type)), start=1):
        if act and t == "int4":
            out[f"packed{k}"] = pack_int4(out[f"code{k}"])
    out["active"] = (a1, a2)
    return out


def rms_norm_dq(x, gamma, beta=None, smooth=None, eps=1e-6, y_type="int8", dtype="fp16",
                want_pre=True):
    """RmsNormDynamicQuant: one input, one quantized output, no xOut."""
    out = _run(x, None, gamma, beta, smooth, None, eps, QMAX[y_type], 0, dtype, False,
               want_pre)
    res = {"code": out["code1"], "scale": out["scale1"]}
    if want_pre:
        res["pre"] = out["pre1"]
    if y_type == "int4":
        res["packed"] = pack_int4(out["code1"])
    return res


def w8a8_gemm_at(a, a_scale, w, w_scale, bias, rows, cols):
    """Outputs (row rows[t], column cols[t]) of the INT8 GEMM with scales:
    returns (exact int64 sums, double outputs)."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    k = a.shape[-1]
    a = a.reshape(-1, k)
    assert w.shape[1] == k
    sa = np.ascontiguousarray(a_scale, dtype=np.float32).reshape(-1)
    sw = np.ascontiguousarray(w_scale, dtype=np.float32).reshape(-1)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32).reshape(-1)
    mi = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    ni = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
    assert mi.size == ni.size
    assert (mi >= 0).all() and (mi < a.shape[0]).all() and (ni >= 0).all() and (ni < w.shape[0]).all()
    sums = np.empty(mi.size, np.int64)
    out = np.empty(mi.size, np.float64)
    if _load().oracle_w8a8_gemm_at(mi.size, _ptr(mi), _ptr(ni), k, _ptr(a), _ptr(sa), _ptr(w),
                                   _ptr(sw), _ptr(b), _ptr(sums), _ptr(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return sums, out


def w8a8_gemm(a, a_scale, w, w_scale, bias=None):
    """Every output of the INT8 GEMM with scales: (sums [m, n], out [m, n])."""
    m = int(np.prod(np.shape(a)[:-1]))
    n = np.shape(w)[0]
    rows = np.repeat(np.arange(m), n)
    cols = np.tile(np.arange(n), m)
    sums, out = w8a8_gemm_at(a, a_scale, w, w_scale, bias, rows, cols)
    return sums.reshape(m, n), out.reshape(m, n)


def add_lora(y, x, weight_b, indices, weight_a=None, layer=0, scale=1.0, y_offset=0,
             dtype="bf16", rows=None, want_pre=True):
    """AddLora ("aclnnAddLora", Formulas) on host arrays of 16-bit storage
    patterns: y [B, h3], x [B, h1], weight_a [W, L, h1, rank] or None,
    weight_b [W, L, rank, h2], indices [B] int32.  Returns (out [n, h3]
    storage patterns, pre [n, h2] slice values before rounding) for the
    requested rows (all when rows is None)."""
    y = np.ascontiguousarray(y, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wb = np.ascontiguousarray(weight_b, dtype=np.uint16)
    wa = None if weight_a is None else np.ascontiguousarray(weight_a, dtype=np.uint16)
    idx = np.ascontiguousarray(indices, dtype=np.int32).reshape(-1)
    nrows, h3 = y.shape
    h1 = x.shape[1]
    w, nl, rank, h2 = wb.shape
    if x.shape[0] != nrows or idx.size != nrows:
        raise ValueError("x, y and indices disagree on the number of rows")
    if wa is not None and wa.shape != (w, nl, h1, rank):
        raise ValueError("weight_a must be [W, L, h1, rank]")
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    n = nrows if sel is None else sel.size
    out = np.empty((n, h3), np.uint16)
    pre = np.empty((n, h2), np.float64) if want_pre else None
    work = np.empty(rank, np.float64)
    rc = _load().oracle_add_lora(
        nrows, h1, rank, h2, h3, w, nl, DTYPES[dtype], _ptr(y), _ptr(x), _ptr(wa), _ptr(wb),
        _ptr(idx), int(layer), float(scale), int(y_offset), n, _ptr(sel), _ptr(out), _ptr(pre),
        _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, pre
