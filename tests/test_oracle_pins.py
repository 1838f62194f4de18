"""Pins for the CPU oracle: checks against things other than the oracle itself.

 - hand-worked rows from the pages' formulas (tests/golden/worked_rows.json);
 - the output-validity truth table of the V2 page (tests/golden/mask_table.json);
 - library routines: numpy's float16 and torch's bfloat16 conversions, and
   torch's rms_norm for the normalisation step;
 - exact-rational / 50-digit brute force on tiny rows;
 - closed forms (constant rows, one-hot rows) and invariants on the
   synthetic workloads.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import check_codes, from_bits, near_tie, to_bits, unpack_int4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed(v):
    val = Fraction(v["frac"])
    if "div_sqrt" in v:
        getcontext().prec = 50
        d = Fraction(v["div_sqrt"])
        val_dec = Decimal(val.numerator) / Decimal(val.denominator)
        return float(val_dec / (Decimal(d.numerator) / Decimal(d.denominator)).sqrt())
    return float(val)


def _run_case(c):
    dt = c["dtype"]
    b = lambda k: None if c.get(k) is None else to_bits(c[k], dt)
    if c["op"] == "v2":
        return oracle.add_rms_norm_dq_v2(
            b("x1"), b("x2"), b("gamma"), b("beta"), b("smooth1"), b("smooth2"), c["eps"],
            c["mask"], c["y_types"][0], c["y_types"][1], dt)
    r = oracle.rms_norm_dq(b("x1"), b("gamma"), b("beta"), b("smooth1"), c["eps"],
                           c["y_types"][0], dt)
    out = {"code1": r["code"], "scale1": r["scale"], "pre1": r["pre"]}
    if "packed" in r:
        out["packed1"] = r["packed"]
    return out


with open(os.path.join(GOLDEN, "worked_rows.json")) as f:
    _CASES = json.load(f)["cases"]


@pytest.mark.parametrize("case", _CASES, ids=[c["name"] for c in _CASES])
def test_worked_rows(case):
    got = _run_case(case)
    exp = case["expect"]
    if "active" in exp:
        assert list(got["active"]) == exp["active"]
    if "x_out" in exp:
        assert np.array_equal(got["x_out"], to_bits(exp["x_out"], case["dtype"]))
    for k in (1, 2):
        if f"scale{k}" not in exp:
            assert f"code{k}" not in got
            continue
        want_scale = np.array([_closed(v) for v in exp[f"scale{k}"]])
        s = got[f"scale{k}"].astype(np.float64)
        # the stored scale is the float nearest the exact value
        assert np.all(np.abs(s - want_scale) <= np.abs(want_scale) * 2.0 ** -24), (s, want_scale)
        want = np.array(exp[f"code{k}"])
        ok = np.array(exp.get("near_tie_ok", np.zeros_like(want, bool)))
        c = got[f"code{k}"].astype(np.int64)
        assert np.all((c == want) | (ok & (np.abs(c - want) <= 1))), (c, want)
        if f"packed{k}" in exp:
            assert np.array_equal(got[f"packed{k}"], np.array(exp[f"packed{k}"], np.uint8))


def test_mask_truth_table():
    with open(os.path.join(GOLDEN, "mask_table.json")) as f:
        rows = json.load(f)["rows"]
    assert len(rows) == 20
    for mask, s1, s2, valid, y1, y2 in rows:
        ok, a1, a2 = oracle.v2_outputs(mask, s1, s2)
        assert ok == valid, (mask, s1, s2)
        if valid:
            assert (a1, a2) == (y1, y2), (mask, s1, s2)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_storage_decode_every_pattern(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = from_bits(bits, dtype)
    got = np.array([oracle.storage_value(int(b), dtype) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _random_doubles(rng, n, lo_exp, hi_exp):
    mant = rng.uniform(1.0, 2.0, n)
    exps = rng.integers(lo_exp, hi_exp, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, exps)


def test_round_to_storage_fp16_matches_numpy():
    rng = np.random.default_rng(11)
    vals = list(_random_doubles(rng, 4000, -27, 17))
    # exact ties between neighbouring fp16 values, normal and subnormal
    h = rng.integers(0, 0x7BFF, 2000).astype(np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals += list((a + b) / 2) + list(-(a + b) / 2)
    vals += [65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001,
             2.0 ** -26, 0.0, -0.0, 5.96e-8, 6.1e-5]
    for v in vals:
        with np.errstate(over="ignore"):  # values past the fp16 range round to inf
            want = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        assert oracle.round_to_storage(v, "fp16") == want, v


def _exact_round(q: Fraction, p: int, emin: int, emax: int):
    """Round a rational to p significant bits, ties to even; None = overflow."""
    if q == 0:
        return Fraction(0)
    m = abs(q)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - p + 1)
    t = m / quantum
    n = math.floor(t)
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (emax + 1):
        return None
    return r if q > 0 else -r


def test_round_to_storage_bf16_matches_exact_and_torch():
    rng = np.random.default_rng(12)
    vals = list(_random_doubles(rng, 3000, -135, 128))
    u = rng.integers(0, 0x7F7F, 2000).astype(np.uint32)
    a = (u << 16).view(np.float32).astype(np.float64)
    b = ((u + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    vals += list((a + b) / 2) + list(-(a + b) / 2)
    for v in vals:
        r = _exact_round(Fraction(v), 8, -126, 127)
        if r is None:
            want = 0x7F80 | (0x8000 if v < 0 else 0)
        else:
            want = int(to_bits([float(r)], "bf16")[0]) if r != 0 else (0x8000 if v < 0 else 0)
        assert oracle.round_to_storage(v, "bf16") == want, v
    # float32-exact inputs: torch's float32 -> bfloat16 conversion (round to nearest even)
    f32 = _random_doubles(rng, 3000, -120, 120).astype(np.float32)
    tb = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, w in zip(f32.astype(np.float64), tb):
        assert oracle.round_to_storage(float(v), "bf16") == int(w), v


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_xout_is_correctly_rounded_sum(dtype):
    """xOut = the sum x1 + x2 rounded once to the storage type, for pairs
    spanning every exponent gap."""
    rng = np.random.default_rng(13)
    n = 4096
    if dtype == "bf16":
        e1 = rng.integers(-30, 30, n)
        e2 = e1 - rng.integers(0, 40, n)
    else:
        e1 = rng.integers(-14, 15, n)
        e2 = np.maximum(e1 - rng.integers(0, 20, n), -24)
    v1 = rng.choice([-1, 1], n) * np.ldexp(rng.uniform(1, 2, n), e1)
    v2 = rng.choice([-1, 1], n) * np.ldexp(rng.uniform(1, 2, n), e2)
    if dtype == "bf16":
        b1 = (v1.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        b2 = (v2.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    else:
        b1 = v1.astype(np.float16).view(np.uint16)
        b2 = v2.astype(np.float16).view(np.uint16)
    x1 = b1.reshape(1, n)
    x2 = b2.reshape(1, n)
    g = to_bits(np.ones(n), dtype)
    out = oracle.add_rms_norm_dq_v2(x1, x2, g, dtype=dtype, want_pre=False)
    f1, f2 = from_bits(b1, dtype), from_bits(b2, dtype)
    p, emin, emax = (8, -126, 127) if dtype == "bf16" else (11, -14, 15)
    for j in range(n):
        r = _exact_round(Fraction(f1[j]) + Fraction(f2[j]), p, emin, emax)
        assert r is not None
        got = from_bits(out["x_out"][0, j], dtype)
        assert got == float(r), (f1[j], f2[j], got, float(r))


def test_rmsnorm_step_matches_torch_rms_norm():
    """With no smooth scale and beta = 0 the quantizer input is
    torch.nn.functional.rms_norm(x, weight=gamma, eps); check the scales and
    the codes against it (float64)."""
    rng = np.random.default_rng(14)
    for dtype, n, eps in (("fp16", 96, 1e-6), ("bf16", 257, 0.5), ("fp16", 1, 1e-3)):
        rows = 5
        x = rng.normal(0, 2, (rows, n))
        g = rng.uniform(0.5, 1.5, n)
        xb = to_bits(x.astype(np.float16) if dtype == "fp16" else
                     (x.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32),
                     dtype)
        gb = to_bits(g.astype(np.float16) if dtype == "fp16" else
                     (g.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32),
                     dtype)
        r = oracle.rms_norm_dq(xb, gb, eps=eps, dtype=dtype)
        xt = torch.from_numpy(from_bits(xb, dtype))
        gt = torch.from_numpy(from_bits(gb, dtype))
        y = torch.nn.functional.rms_norm(xt, (n,), weight=gt, eps=float(np.float32(eps)))
        m = y.abs().amax(dim=1).numpy()
        want_scale = (m / 127.0).astype(np.float32)
        assert np.all(np.abs(r["scale"].astype(np.float64) - want_scale) <=
                      np.abs(want_scale) * 2.0 ** -23)
        v = y.numpy() / r["scale"].astype(np.float64)[:, None]
        assert np.allclose(r["pre"], v, rtol=1e-12, atol=1e-12)
        check_codes(r["code"], np.clip(np.rint(v), -127, 127), v, tol=1e-9)


def _brute_row(a1, a2, g, b, s1, s2, eps, qs):
    """Exact rationals for the sum, 60-digit decimals after the square root."""
    getcontext().prec = 60
    n = len(a1)
    a = [Fraction(float(u)) + (Fraction(float(v)) if a2 is not None else 0)
         for u, v in zip(a1, a2 if a2 is not None else a1)]
    ss = sum(t * t for t in a)
    ms = ss / n + Fraction(float(np.float32(eps)))
    dec = lambda fr: Decimal(fr.numerator) / Decimal(fr.denominator)
    rms = dec(ms).sqrt()
    y = [dec(a[j]) / rms * Decimal(float(g[j])) + (Decimal(float(b[j])) if b is not None else 0)
         for j in range(n)]
    res = []
    for s, q in zip((s1, s2), qs):
        if q == 0:
            res.append(None)
            continue
        inp = [y[j] * Decimal(float(s[j])) if s is not None else y[j] for j in range(n)]
        m = max(abs(t) for t in inp)
        scale = np.float32(float(m / q))
        v = [float(t / Decimal(float(scale))) if scale != 0 else 0.0 for t in inp]
        res.append((scale, np.array(v)))
    return res


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_rows(seed):
    rng = np.random.default_rng(100 + seed)
    dtype = "bf16" if seed % 2 else "fp16"
    n = 2 * int(rng.integers(1, 17))  # INT4 output needs an even row length
    rows = 3
    w = synth.Workload("tiny", "v2", rows, n, dtype, 1000 + seed, (True, True), True, 2,
                       ("int8", "int4") if seed % 3 == 0 else ("int4", "int8"))
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    eps = [1e-6, 0.1, 0.0][seed % 3]
    out = oracle.add_rms_norm_dq_v2(x1, x2, g, b, s1, s2, eps, (True, True), *w.y_types,
                                    dtype=dtype)
    qs = [oracle.QMAX[t] for t in w.y_types]
    fx1, fx2 = from_bits(x1, dtype), from_bits(x2, dtype)
    fg, fb, f1, f2 = (from_bits(t, dtype) for t in (g, b, s1, s2))
    for i in range(rows):
        res = _brute_row(fx1[i], fx2[i], fg, fb, f1, f2, eps, qs)
        for k, r in enumerate(res, start=1):
            scale, v = r
            assert out[f"scale{k}"][i] == scale
            assert np.allclose(out[f"pre{k}"][i], v, rtol=1e-12, atol=1e-12)
            check_codes(out[f"code{k}"][i], np.clip(np.rint(v), -qs[k - 1], qs[k - 1]), v,
                        tol=1e-9)


def test_closed_form_constant_and_one_hot_rows():
    n = 64
    ones = to_bits(np.ones(n), "bf16")
    # constant row c: y = sign(c), scale 1/127, codes +-127
    for c in (0.75, -3.0, 1024.0):
        x1 = to_bits(np.full((1, n), c), "bf16")
        x2 = to_bits(np.zeros((1, n)), "bf16")
        o = oracle.add_rms_norm_dq_v2(x1, x2, ones, eps=0.0)
        assert abs(float(o["scale1"][0]) - 1 / 127) <= 2.0 ** -24 / 127 * 2
        assert np.all(o["code1"] == (127 if c > 0 else -127))
    # one-hot row a*e_k with n = 64: y_k = 8*sign(a), scale 8/127
    for a, k in ((2.5, 3), (-0.125, 63), (96.0, 0)):
        x = np.zeros((1, n))
        x[0, k] = a
        o = oracle.add_rms_norm_dq_v2(to_bits(x, "bf16"), to_bits(np.zeros((1, n)), "bf16"),
                                      ones, eps=0.0)
        assert float(o["scale1"][0]) == np.float32(8.0 / 127.0)
        want = np.zeros(n, np.int8)
        want[k] = 127 if a > 0 else -127
        assert np.array_equal(o["code1"][0], want)


def test_pack_int4_nibble_order():
    codes = np.array([[-8, 7, 1, -1, 0, -7, 3, 4]], np.int8)
    p = oracle.pack_int4(codes)
    assert p.tolist() == [[0x78, 0xF1, 0x90, 0x43]]
    assert np.array_equal(unpack_int4(p), codes)


def _invariants(code, scale, pre, q):
    pre = pre.astype(np.float64)
    scale = scale.astype(np.float64)
    nz = scale > 0
    assert np.all(np.abs(code[nz]).max(axis=1) == q)
    inp = pre * scale[:, None]
    err = np.abs(code * scale[:, None] - inp)
    assert np.all(err <= scale[:, None] / 2 * (1 + 1e-6) + 1e-30)
    assert np.all((np.sign(code) == np.sign(inp)) | (code == 0))
    for i in range(code.shape[0]):
        order = np.argsort(inp[i], kind="stable")
        assert np.all(np.diff(code[i][order].astype(np.int32)) >= 0)


@pytest.mark.parametrize("name,rows", [("rmsnorm_dq", None), ("v2_square", 24),
                                       ("v2_decode", 4), ("v2_outlier", 4), ("v2_int4", 16)])
def test_invariants_on_workloads(name, rows):
    w = synth.WORKLOADS[name]
    x1, x2 = synth.inputs(w, rows=rows)
    g, b, s1, s2 = synth.params(w)
    if w.op == "rmsnorm":
        r = oracle.rms_norm_dq(x1, g, b, s1, w.eps, w.y_types[0], w.dtype)
        _invariants(r["code"], r["scale"], r["pre"], oracle.QMAX[w.y_types[0]])
        return
    o = oracle.add_rms_norm_dq_v2(x1, x2, g, b, s1, s2, w.eps, w.mask, *w.y_types,
                                  dtype=w.dtype)
    for k in (1, 2):
        if o["active"][k - 1]:
            _invariants(o[f"code{k}"], o[f"scale{k}"], o[f"pre{k}"],
                        oracle.QMAX[w.y_types[k - 1]])
    # near-tie codes are rare on these inputs
    assert near_tie(o["pre1"], 1e-3).mean() < 0.01


# ---- the consumer GEMM of the codes ------------------------------------------

def test_gemm_worked_example():
    with open(os.path.join(GOLDEN, "gemm_worked.json")) as f:
        c = json.load(f)
    sums, out = oracle.w8a8_gemm(np.array(c["a"]), np.array(c["a_scale"]), np.array(c["w"]),
                                 np.array(c["w_scale"]), np.array(c["bias"]))
    assert sums.tolist() == c["sums"]
    assert out.tolist() == c["out"]


def test_gemm_sums_match_numpy_integer_matmul():
    rng = np.random.default_rng(21)
    for m, n, k in ((3, 5, 16), (17, 9, 48), (8, 33, 160)):
        a = rng.integers(-127, 128, (m, k)).astype(np.int8)
        w = rng.integers(-127, 128, (n, k)).astype(np.int8)
        sa = rng.uniform(0.01, 1, m).astype(np.float32)
        sw = rng.uniform(0.01, 1, n).astype(np.float32)
        b = rng.normal(0, 1, n).astype(np.float32)
        sums, out = oracle.w8a8_gemm(a, sa, w, sw, b)
        ref = a.astype(np.int64) @ w.astype(np.int64).T
        assert np.array_equal(sums, ref)
        want = ref * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] + b
        assert np.allclose(out, want, rtol=1e-15, atol=1e-12)


def test_gemm_scaled_identity_closed_form():
    """w = c * identity: out[m, j] = a[m, j] * c * a_scale[m] * w_scale[j]."""
    rng = np.random.default_rng(22)
    k = 32
    a = rng.integers(-127, 128, (6, k)).astype(np.int8)
    w = (np.eye(k) * 3).astype(np.int8)
    sa = rng.uniform(0.1, 1, 6).astype(np.float32)
    sw = rng.uniform(0.1, 1, k).astype(np.float32)
    sums, out = oracle.w8a8_gemm(a, sa, w, sw)
    assert np.array_equal(sums, 3 * a.astype(np.int64))
    assert np.allclose(out, 3.0 * a * sa[:, None].astype(np.float64) * sw[None, :], rtol=1e-15)
