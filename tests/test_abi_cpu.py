"""Host-side checks of the C-ABI library that need no GPU.

 - the library loads and exports every function include/adq.h declares;
 - phase-1 validation: every error status, and the output-mask truth table
   of the V2 page (Formula cases + Constraints), driven through the C-ABI
   with placeholder device addresses.  No kernel is launched: phase 1 only
   inspects descriptors.  On a machine without a GPU a well-formed call ends
   in ADQ_ERR_RUNTIME ("no HIP device"); with one it returns ADQ_OK and an
   executor, which is destroyed without running.
"""
import ctypes
import json
import os
import re

import pytest

import int4_dynamic_quantization_amd as adq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ACCEPTED = (adq.OK, adq.ERR_RUNTIME)

# placeholder device addresses, 256-byte aligned and distinct
_next = [0x10000000]


def fake(shape, dtype):
    t = adq.Tensor()
    t.data = _next[0]
    _next[0] += 1 << 24
    t.dtype = dtype
    t.ndim = len(shape)
    for i, s in enumerate(shape):
        t.shape[i] = s
    return t


def declared_functions():
    with open(os.path.join(ROOT, "include", "adq.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(adq_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 14, names
    assert set(names) == set(adq.EXPORTED)
    for name in names:
        assert hasattr(adq.lib, name), name
    # and the symbols come from this library, not a loaded dependency
    handle = ctypes.CDLL(adq.LIB_PATH)
    for name in names:
        assert ctypes.cast(getattr(handle, name), ctypes.c_void_p).value


def v2_call(x1=None, x2=None, gamma=None, beta=None, s1=None, s2=None, eps=1e-6, mask=None,
            y1=None, y2=None, sc1=None, sc2=None, xo=None, out_ptrs=True):
    m = None if mask is None else (ctypes.c_bool * 2)(*mask)
    ws = ctypes.c_uint64(0)
    ex = ctypes.c_void_p(None)
    r = lambda t: None if t is None else ctypes.byref(t)
    st = adq.lib.adq_add_rms_norm_dynamic_quant_v2_get_workspace_size(
        r(x1), r(x2), r(gamma), r(beta), r(s1), r(s2), eps, m, r(y1), r(y2), r(sc1), r(sc2),
        r(xo), ctypes.byref(ws) if out_ptrs else None, ctypes.byref(ex) if out_ptrs else None)
    if ex.value:
        adq.lib.adq_executor_destroy(ex)
    return st


def full_v2(M=4, N=64, dt=adq.BF16, q1=adq.INT8, q2=adq.INT8, smooth=2):
    n1 = N // 2 if q1 == adq.INT4X2 else N
    n2 = N // 2 if q2 == adq.INT4X2 else N
    return dict(
        x1=fake([M, N], dt), x2=fake([M, N], dt), gamma=fake([N], dt), beta=fake([N], dt),
        s1=fake([N], dt) if smooth >= 1 else None, s2=fake([N], dt) if smooth >= 2 else None,
        y1=fake([M, n1], q1), y2=fake([M, n2], q2), sc1=fake([M], adq.F32),
        sc2=fake([M], adq.F32), xo=fake([M, N], dt))


def test_valid_call_accepted():
    assert v2_call(**full_v2()) in ACCEPTED
    assert v2_call(**full_v2(dt=adq.F16, q1=adq.INT4X2)) in ACCEPTED
    # leading dims flattened, scale with shape [...]
    a = full_v2()
    a.update(x1=fake([2, 3, 64], adq.BF16), x2=fake([2, 3, 64], adq.BF16),
             xo=fake([2, 3, 64], adq.BF16), y1=fake([2, 3, 64], adq.INT8),
             y2=fake([2, 3, 64], adq.INT8), sc1=fake([2, 3], adq.F32), sc2=fake([6], adq.F32))
    assert v2_call(**a) in ACCEPTED


def test_mask_truth_table_through_phase_one():
    with open(os.path.join(ROOT, "tests", "golden", "mask_table.json")) as f:
        rows = json.load(f)["rows"]
    for mask, has1, has2, valid, y1, y2 in rows:
        a = full_v2()
        if not has1:
            a["s1"] = None
        if not has2:
            a["s2"] = None
        st = v2_call(mask=mask, **a)
        if not valid:
            assert st == adq.ERR_PARAM_INVALID, (mask, has1, has2, adq.last_error())
            continue
        assert st in ACCEPTED, (mask, has1, has2, adq.last_error())
        # an output that is produced is required; one that is not may be NULL
        for k, active in ((1, y1), (2, y2)):
            b = dict(a)
            b[f"y{k}"] = None
            st = v2_call(mask=mask, **b)
            if active:
                assert st == adq.ERR_NULLPTR, (mask, has1, has2, k)
            else:
                assert st in ACCEPTED, (mask, has1, has2, k, adq.last_error())


@pytest.mark.parametrize("out,src", [("xo", "x1"), ("xo", "x2"), ("y1", "x1"), ("sc1", "gamma"),
                                     ("y2", "s2"), ("y2", "y1"), ("sc2", "xo")])
def test_outputs_sharing_memory_rejected(out, src):
    """A produced output overlapping an input or another produced output
    (same start, or a range that reaches into it) is rejected."""
    for shift in (0, 3):
        a = full_v2()
        a[out].data = a[src].data + shift
        assert v2_call(**a) == adq.ERR_PARAM_INVALID, (out, src, shift)
        assert "share" in adq.last_error() and "memory" in adq.last_error()
    # an output that is not produced may sit anywhere
    a = full_v2(smooth=1)
    a["y2"].data = a["x1"].data
    assert v2_call(mask=(True, False), **a) in ACCEPTED


@pytest.mark.parametrize("field", ["x1", "x2", "gamma", "xo"])
def test_required_tensor_missing(field):
    a = full_v2()
    a[field] = None
    assert v2_call(**a) == adq.ERR_NULLPTR


def test_null_data_pointer_and_out_pointers():
    a = full_v2()
    a["gamma"].data = None
    assert v2_call(**a) == adq.ERR_NULLPTR
    assert v2_call(out_ptrs=False, **full_v2()) == adq.ERR_NULLPTR


@pytest.mark.parametrize("field", ["x1", "x2", "xo", "gamma", "y1", "sc1"])
def test_empty_tensor_rejected(field):
    a = full_v2()
    t = a[field]
    t.shape[0] = 0
    assert v2_call(**a) == adq.ERR_PARAM_INVALID
    assert "empty" in adq.last_error()


@pytest.mark.parametrize("shape", [[1 << 32, 1 << 32, 64], [1 << 40, 1 << 7]])
def test_huge_element_counts_rejected(shape):
    """Shapes whose element count overflows int64 (or exceeds 2^46) are
    refused in phase 1, before any size is computed from them."""
    a = full_v2()
    for f in ("x1", "x2", "xo"):
        a[f] = fake(shape, a[f].dtype)
    assert v2_call(**a) == adq.ERR_PARAM_INVALID
    assert "2^46" in adq.last_error()


def test_shape_and_dtype_mismatches():
    cases = []
    a = full_v2(); a["x2"] = fake([4, 32], adq.BF16); cases.append(a)
    a = full_v2(); a["x2"] = fake([4, 64], adq.F16); cases.append(a)
    a = full_v2(); a["xo"] = fake([4, 64], adq.F16); cases.append(a)
    a = full_v2(); a["gamma"] = fake([63], adq.BF16); cases.append(a)
    a = full_v2(); a["beta"] = fake([64], adq.F16); cases.append(a)
    a = full_v2(); a["s2"] = fake([1, 64], adq.BF16); cases.append(a)
    a = full_v2(); a["y1"] = fake([4, 32], adq.INT8); cases.append(a)
    a = full_v2(); a["y2"] = fake([4, 64], adq.INT4X2); cases.append(a)
    a = full_v2(); a["y1"] = fake([3, 64], adq.INT8); cases.append(a)
    a = full_v2(); a["sc1"] = fake([5], adq.F32); cases.append(a)
    a = full_v2(); a["sc2"] = fake([4], adq.F16); cases.append(a)
    for i, c in enumerate(cases):
        assert v2_call(**c) == adq.ERR_PARAM_INVALID, (i, adq.last_error())


def test_odd_width_int4_rejected():
    a = full_v2(N=63, q1=adq.INT4X2)
    a["y1"] = fake([4, 31], adq.INT4X2)
    assert v2_call(**a) == adq.ERR_PARAM_INVALID
    # INT8 accepts odd widths (generic kernel)
    assert v2_call(**full_v2(N=63)) in ACCEPTED


def test_unsupported_dtypes():
    a = full_v2()
    for t in ("x1", "x2", "xo"):
        a[t] = fake([4, 64], adq.F32)
    assert v2_call(**a) == adq.ERR_UNSUPPORTED
    a = full_v2()
    a["y1"] = fake([4, 64], adq.F16)
    assert v2_call(**a) == adq.ERR_UNSUPPORTED


def test_bad_epsilon():
    assert v2_call(eps=float("nan"), **full_v2()) == adq.ERR_PARAM_INVALID
    assert v2_call(eps=float("inf"), **full_v2()) == adq.ERR_PARAM_INVALID


def rms_call(x, gamma, beta, smooth, y, sc, eps=1e-6):
    ws = ctypes.c_uint64(0)
    ex = ctypes.c_void_p(None)
    r = lambda t: None if t is None else ctypes.byref(t)
    st = adq.lib.adq_rms_norm_dynamic_quant_get_workspace_size(
        r(x), r(gamma), r(beta), r(smooth), eps, r(y), r(sc), ctypes.byref(ws), ctypes.byref(ex))
    if ex.value:
        adq.lib.adq_executor_destroy(ex)
    return st


def test_rms_norm_dq_validation():
    x, g = fake([64, 1024], adq.F16), fake([1024], adq.F16)
    y, sc = fake([64, 1024], adq.INT8), fake([64], adq.F32)
    assert rms_call(x, g, None, None, y, sc) in ACCEPTED
    assert rms_call(x, g, None, fake([1024], adq.F16), fake([64, 512], adq.INT4X2),
                    sc) in ACCEPTED
    assert rms_call(x, None, None, None, y, sc) == adq.ERR_NULLPTR
    assert rms_call(x, g, None, None, None, sc) == adq.ERR_NULLPTR
    assert rms_call(x, g, None, None, y, None) == adq.ERR_NULLPTR
    assert rms_call(x, fake([1024], adq.BF16), None, None, y, sc) == adq.ERR_PARAM_INVALID
    assert rms_call(fake([0, 1024], adq.F16), g, None, None, y, sc) == adq.ERR_PARAM_INVALID
    assert rms_call(x, g, None, None, fake([64, 1024], adq.F32), sc) == adq.ERR_UNSUPPORTED


def test_phase_two_and_helpers_reject_null_executor():
    assert adq.lib.adq_add_rms_norm_dynamic_quant_v2(None, 0, None, None) == adq.ERR_NULLPTR
    assert adq.lib.adq_rms_norm_dynamic_quant(None, 0, None, None) == adq.ERR_NULLPTR
    ws = ctypes.c_uint64(0)
    assert adq.lib.adq_executor_set_path(None, 0, ctypes.byref(ws)) == adq.ERR_NULLPTR
    assert adq.lib.adq_executor_describe(None, None, 0) == -1
    adq.lib.adq_executor_destroy(None)
    assert isinstance(adq.last_error(), str)


def gemm_call(a, sa, w, sw, bias, out, out_ptrs=True):
    ws = ctypes.c_uint64(0)
    ex = ctypes.c_void_p(None)
    r = lambda t: None if t is None else ctypes.byref(t)
    st = adq.lib.adq_w8a8_gemm_get_workspace_size(
        r(a), r(sa), r(w), r(sw), r(bias), r(out), ctypes.byref(ws) if out_ptrs else None,
        ctypes.byref(ex) if out_ptrs else None)
    if ex.value:
        adq.lib.adq_executor_destroy(ex)
    return st


def full_gemm(m=64, n=48, k=128, out=adq.BF16):
    return dict(a=fake([m, k], adq.INT8), sa=fake([m], adq.F32), w=fake([n, k], adq.INT8),
                sw=fake([n], adq.F32), bias=fake([n], adq.F32), out=fake([m, n], out))


def test_gemm_valid_calls():
    for out in (adq.F32, adq.BF16, adq.F16):
        assert gemm_call(**full_gemm(out=out)) in ACCEPTED, adq.last_error()
    a = full_gemm()
    a["bias"] = None
    assert gemm_call(**a) in ACCEPTED
    a = full_gemm()
    a.update(a=fake([2, 32, 128], adq.INT8), sa=fake([2, 32], adq.F32),
             out=fake([2, 32, 48], adq.BF16))
    assert gemm_call(**a) in ACCEPTED


def test_gemm_validation():
    for f in ("a", "sa", "w", "sw", "out"):
        a = full_gemm()
        a[f] = None
        assert gemm_call(**a) == adq.ERR_NULLPTR, f
    assert gemm_call(out_ptrs=False, **full_gemm()) == adq.ERR_NULLPTR
    bad = []
    a = full_gemm(k=120); a["w"] = fake([48, 120], adq.INT8); bad.append(a)  # k % 16
    a = full_gemm(k=(1 << 17) + 16); bad.append(a)                            # k too large
    a = full_gemm(); a["w"] = fake([48, 64], adq.INT8); bad.append(a)         # k mismatch
    a = full_gemm(); a["sa"] = fake([63], adq.F32); bad.append(a)
    a = full_gemm(); a["sw"] = fake([47], adq.F32); bad.append(a)
    a = full_gemm(); a["bias"] = fake([1, 48], adq.F32); bad.append(a)
    a = full_gemm(); a["out"] = fake([64, 47], adq.BF16); bad.append(a)
    a = full_gemm(); a["out"] = fake([63, 48], adq.BF16); bad.append(a)
    a = full_gemm(); a["a"].data += 8; bad.append(a)                           # alignment
    a = full_gemm(); a["sa"].data += 2; bad.append(a)
    a = full_gemm(); a["out"].shape[0] = 0; bad.append(a)
    for i, c in enumerate(bad):
        assert gemm_call(**c) == adq.ERR_PARAM_INVALID, (i, adq.last_error())
    unsupported = []
    a = full_gemm(); a["a"] = fake([64, 128], adq.F16); unsupported.append(a)
    a = full_gemm(); a["sw"] = fake([48], adq.BF16); unsupported.append(a)
    a = full_gemm(); a["out"] = fake([64, 48], adq.INT8); unsupported.append(a)
    for i, c in enumerate(unsupported):
        assert gemm_call(**c) == adq.ERR_UNSUPPORTED, (i, adq.last_error())
    assert adq.lib.adq_w8a8_gemm(None, 0, None, None) == adq.ERR_NULLPTR


def lora_call(y, x, wb, idx, wa, layer=1, scale=0.5, off=0, size=None, out=None,
              out_ptrs=True):
    ws = ctypes.c_uint64(0)
    ex = ctypes.c_void_p(None)
    r = lambda t: None if t is None else ctypes.byref(t)
    size = (wb.shape[3] if wb is not None else 96) if size is None else size
    st = adq.lib.adq_add_lora_get_workspace_size(
        r(y), r(x), r(wb), r(idx), r(wa), layer, scale, off, size, r(out),
        ctypes.byref(ws) if out_ptrs else None, ctypes.byref(ex) if out_ptrs else None)
    if ex.value:
        adq.lib.adq_executor_destroy(ex)
    return st


def full_lora(rows=64, h1=128, rank=16, h2=96, h3=256, w=4, layers=3, dt=adq.BF16):
    return dict(y=fake([rows, h3], dt), x=fake([rows, h1], dt), wb=fake([w, layers, rank, h2], dt),
                idx=fake([rows], adq.INT32), wa=fake([w, layers, h1, rank], dt),
                out=fake([rows, h3], dt))


def test_lora_valid_calls():
    assert lora_call(**full_lora()) in ACCEPTED, adq.last_error()
    assert lora_call(**full_lora(dt=adq.F16)) in ACCEPTED, adq.last_error()
    a = full_lora(h1=16)
    a["wa"] = None  # no shrink: h1 == rank
    assert lora_call(**a) in ACCEPTED, adq.last_error()
    a = full_lora()
    a["out"] = a["y"]  # in place
    assert lora_call(**a) in ACCEPTED
    a = full_lora()
    a.update(y=fake([2, 32, 256], adq.BF16), x=fake([2, 32, 128], adq.BF16),
             out=fake([2, 32, 256], adq.BF16), idx=fake([2, 32], adq.INT32))
    assert lora_call(**a) in ACCEPTED
    assert lora_call(off=160, **full_lora()) in ACCEPTED  # slice ends at h3


def test_lora_validation():
    for f in ("y", "x", "wb", "idx", "out"):
        a = full_lora()
        a[f] = None
        assert lora_call(**a) == adq.ERR_NULLPTR, f
    assert lora_call(out_ptrs=False, **full_lora()) == adq.ERR_NULLPTR
    bad = []
    bad.append(dict(full_lora(), off=161))                                  # slice past h3
    bad.append(dict(full_lora(), off=-1))
    bad.append(dict(full_lora(), size=95))                                  # slice size != h2
    bad.append(dict(full_lora(), layer=3))                                  # layer out of range
    bad.append(dict(full_lora(), layer=-1))
    bad.append(dict(full_lora(), scale=float("nan")))
    a = full_lora(); a["wa"] = None; bad.append(a)                          # h1 != rank
    a = full_lora(); a["wa"] = fake([4, 3, 128, 8], adq.BF16); bad.append(a)
    a = full_lora(); a["wb"] = fake([4, 3, 16], adq.BF16); bad.append(a)
    a = full_lora(); a["idx"] = fake([63], adq.INT32); bad.append(a)
    a = full_lora(); a["x"] = fake([63, 128], adq.BF16); bad.append(a)
    a = full_lora(); a["out"] = fake([64, 255], adq.BF16); bad.append(a)
    a = full_lora(); a["x"] = fake([64, 128], adq.F16); bad.append(a)       # dtype mismatch
    a = full_lora(); a["y"].shape[0] = 0; bad.append(a)
    for i, c in enumerate(bad):
        assert lora_call(**c) == adq.ERR_PARAM_INVALID, (i, adq.last_error())
    uns = []
    a = full_lora(); a["idx"] = fake([64], adq.INT8); uns.append(a)
    a = full_lora(); a.update(y=fake([64, 256], adq.F32), x=fake([64, 128], adq.F32),
                              out=fake([64, 256], adq.F32)); uns.append(a)
    a = full_lora(w=2049); uns.append(a)
    for i, c in enumerate(uns):
        assert lora_call(**c) == adq.ERR_UNSUPPORTED, (i, adq.last_error())
    assert adq.lib.adq_add_lora(None, 0, None, None) == adq.ERR_NULLPTR
