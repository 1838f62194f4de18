"""Seeded random sweeps on the GPU: many small, irregular calls of each
operation checked against the oracle, beyond the hand-picked shapes of the
other GPU tests.

 - AddRmsNormDynamicQuantV2 / RmsNormDynamicQuant: random row counts, row
   lengths (multiples of 8 up to 16384 columns, rows of 16392..24576 columns
   for the row kernel's four-vectors-per-thread instances, and arbitrary
   lengths for the generic kernel), dtypes,
   valid output-option combinations, INT8/INT4 outputs, beta present or not,
   outlier columns; compared under the parity rules.
 - W8A8 GEMM: random m, n and k (a multiple of 16), output dtype and bias;
   with unit scales, no bias and fp32 output bit-exact integer sums, else the
   bound derived in test_gemm_gpu.py.
 - AddLora: random rows, h1, rank, h2, slice offset, adapters, layers, in
   place or not, with or without weightA, on small-integer data with a
   power-of-two scale, where every fp32 step is exact: bit-exact.

The random parameters come from numpy generators with fixed seeds, so every
run draws the same cases; each case prints its parameters first.
"""
import json
import os

import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import oracle
import synth
from gpu_helpers import compare_rms, compare_v2, oracle_v2, run_rms, run_v2
from test_gemm_gpu import check_scaled, run_gemm
from test_lora_gpu import run_lora, small_ints

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

with open(os.path.join(GOLDEN, "mask_table.json")) as f:
    _VALID = [r for r in json.load(f)["rows"] if r[3]]  # [mask, has_s1, has_s2, valid, ...]


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _row_length(rng):
    kind = rng.integers(0, 4)
    if kind == 0:
        return int(rng.integers(1, 2049)) * 8          # row kernel
    if kind == 1:
        return int(rng.integers(1, 5000))              # any length: generic kernel
    if kind == 2:
        return int(rng.integers(2049, 3073)) * 8       # longer rows: four vectors per thread
    return int(rng.integers(1, 64)) * 8                # short rows


def _v2_case(i):
    rng = np.random.default_rng(9000 + i)
    n = _row_length(rng)
    m = int(rng.integers(1, 120 if n > 8192 else 300))
    dtype = "bf16" if rng.integers(0, 2) else "fp16"
    mask, has1, has2 = _VALID[int(rng.integers(0, len(_VALID)))][:3]
    y_types = tuple("int4" if (n % 2 == 0 and rng.integers(0, 2)) else "int8" for _ in range(2))
    beta = bool(rng.integers(0, 2))
    outlier = 0.01 if rng.integers(0, 3) == 0 else 0.0
    eps = [1e-6, 1e-5, 1e-3][int(rng.integers(0, 3))]
    return dict(m=m, n=n, dtype=dtype, mask=mask, has1=has1, has2=has2, y_types=y_types,
                beta=beta, outlier=outlier, eps=eps, seed=9000 + i)


@pytest.mark.parametrize("i", range(40))
def test_random_v2(i):
    c = _v2_case(i)
    _announce(f"v2 {c}")
    w = synth.Workload("rand", "v2", c["m"], c["n"], c["dtype"], c["seed"], None, c["beta"], 2,
                       outlier_frac=c["outlier"])
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    s1 = s1 if c["has1"] else None
    s2 = s2 if c["has2"] else None
    mask = None if c["mask"] is None else tuple(c["mask"])
    outs, desc = run_v2(x1, x2, g, b, s1, s2, c["eps"], mask, c["y_types"], c["dtype"])
    ora = oracle_v2(x1, x2, g, b, s1, s2, c["eps"], mask, c["y_types"], c["dtype"])
    compare_v2(outs, ora, c["y_types"])
    for k in (1, 2):
        if not ora["active"][k - 1]:
            assert outs[f"y{k}"] is None, desc


@pytest.mark.parametrize("i", range(12))
def test_random_rms_norm_dq(i):
    rng = np.random.default_rng(9500 + i)
    n = _row_length(rng)
    m = int(rng.integers(1, 120 if n > 8192 else 300))
    dtype = "bf16" if rng.integers(0, 2) else "fp16"
    y_type = "int4" if (n % 2 == 0 and rng.integers(0, 2)) else "int8"
    beta, smooth = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    _announce(f"rms m={m} n={n} {dtype} {y_type} beta={beta} smooth={smooth}")
    w = synth.Workload("rand", "rmsnorm", m, n, dtype, 9500 + i, None, beta, int(smooth))
    x, _ = synth.inputs(w)
    g, b, s1, _ = synth.params(w)
    outs, desc = run_rms(x, g, b, s1, 1e-6, y_type, dtype)
    ora = oracle.rms_norm_dq(x, g, b, s1, 1e-6, y_type, dtype)
    compare_rms(outs, ora, y_type)


@pytest.mark.parametrize("i", range(24))
def test_random_gemm(i):
    rng = np.random.default_rng(9700 + i)
    m, n = int(rng.integers(1, 700)), int(rng.integers(1, 700))
    k = int(rng.integers(1, 41)) * 16
    exact = i % 2 == 0
    out = "f32" if exact else ["bf16", "fp16", "f32"][int(rng.integers(0, 3))]
    has_bias = (not exact) and bool(rng.integers(0, 2))
    _announce(f"gemm m={m} n={n} k={k} out={out} bias={has_bias} exact={exact}")
    a = rng.integers(-127, 128, (m, k)).astype(np.int8)
    w = rng.integers(-127, 128, (n, k)).astype(np.int8)
    if exact:
        sa, sw, bias = np.ones(m, np.float32), np.ones(n, np.float32), None
    else:
        sa = rng.uniform(0.01, 0.08, m).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-3, n).astype(np.float32)
        bias = rng.normal(0, 0.1, n).astype(np.float32) if has_bias else None
    got, desc = run_gemm(a, sa, w, sw, bias, out=out)
    sums, ref = oracle.w8a8_gemm(a, sa, w, sw, bias)
    if exact:
        assert np.array_equal(got, sums.astype(np.float32)), desc
    else:
        check_scaled(got, sums, ref, sa[:, None], sw[None, :],
                     None if bias is None else bias[None, :], out)


@pytest.mark.parametrize("i", range(24))
def test_random_lora(i):
    rng = np.random.default_rng(9900 + i)
    dt = "bf16" if rng.integers(0, 2) else "fp16"
    has_a = bool(rng.integers(0, 4))  # mostly with weightA
    rank = [16, 32, 64, 5, 8, 16, 128, 24][int(rng.integers(0, 8))]
    h1 = (int(rng.integers(1, 65)) * 8 if rng.integers(0, 3) else int(rng.integers(1, 400))) \
        if has_a else rank
    h2 = int(rng.integers(1, 300))
    off = int(rng.integers(0, 80))
    h3 = off + h2 + int(rng.integers(0, 80))
    rows = int(rng.integers(1, 800))
    w, layers = int(rng.integers(1, 10)), int(rng.integers(1, 4))
    layer = int(rng.integers(0, layers))
    in_place = bool(rng.integers(0, 2))
    _announce(f"lora rows={rows} h1={h1} rank={rank} h2={h2} h3={h3} off={off} w={w} "
              f"layers={layers} layer={layer} has_a={has_a} in_place={in_place} {dt}")
    s = 9900 + i
    x = small_ints(s, 12, (rows, h1), -2, 2, dt)
    y = small_ints(s, 13, (rows, h3), -8, 8, dt)
    wa = small_ints(s, 14, (w, layers, h1, rank), -2, 2, dt) if has_a else None
    wb = small_ints(s, 15, (w, layers, rank, h2), -2, 2, dt)
    idx = synth.int32s(s, 16, -1, w, rows)
    got, desc = run_lora(y, x, wa, wb, idx, layer, 0.5, off, dt, in_place=in_place)
    ref, _ = oracle.add_lora(y, x, wb, idx, wa, layer, 0.5, off, dt)
    assert np.array_equal(got, ref), desc
