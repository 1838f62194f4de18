"""Parity of the INT8 GEMM (the consumer of y1Out / scale1Out) with the oracle.

out[m, n] = (sum_k a[m, k] * w[n, k]) * a_scale[m] * w_scale[n] (+ bias[n]).

Bars:
 - integer sums: with unit scales, no bias and float32 output the result is
   the exact sum whenever |sum| <= 2^24, so those cases are compared
   bit-exactly with the oracle's int64 sums;
 - scaled outputs: the kernel forms the value in float32 (at most four
   roundings of unit 2^-24 on |sum * a_scale * w_scale| + |bias|) and then
   rounds it once to the output type (unit u_s: 2^-8 bf16, 2^-11 fp16, plus
   half the fp16 subnormal spacing), so
       |got - exact| <= 5 * 2^-24 * (|P| + |bias|) + u_s * |exact| + sub
   with exact = the oracle's double result;
 - every output is written (outputs are pre-filled with NaN).
Shapes span several tiles of every tile size, ragged M, N and K (K a
multiple of 16), leading dimensions, the full projection size
16384 x 8192 x 8192 and the few-row projections that follow decode-sized
batches (1 to 200 rows of 8192 x 8192) on sampled outputs.
"""
import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
UNIT = {"f32": 0.0, "bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
SUB = {"f32": 2.0 ** -150, "bf16": 2.0 ** -134, "fp16": 2.0 ** -25}


def codes(seed, tid, rows, cols, lo=-127, hi=127):
    return synth.int8_codes(seed, tid, rows, cols, lo, hi)


TILES = [adq.PATH_GEMM_TILE128, adq.PATH_GEMM_TILE256, adq.PATH_GEMM_TILE32]
TILE_IDS = ["tile128", "tile256", "tile32"]
TILE_SIZE = {adq.PATH_GEMM_TILE128: 128, adq.PATH_GEMM_TILE256: 256, adq.PATH_GEMM_TILE32: 32}


def run_gemm(a, sa, w, sw, bias=None, out="bf16", lead=None, path=adq.PATH_AUTO):
    """Run the GEMM through the C-ABI on host arrays; returns (out, describe)."""
    ta = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    if lead is not None:
        ta = ta.reshape(*lead, a.shape[-1])
    tsa = torch.from_numpy(np.ascontiguousarray(sa, dtype=np.float32)).to("cuda")
    tw = torch.from_numpy(np.ascontiguousarray(w)).to("cuda")
    tsw = torch.from_numpy(np.ascontiguousarray(sw, dtype=np.float32)).to("cuda")
    tb = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(
        "cuda")
    o = torch.full(tuple(ta.shape[:-1]) + (w.shape[0],), float("nan"), dtype=OUT_DT[out],
                   device="cuda")
    ex, o = adq.plan_w8a8_gemm(ta, tsa, tw, tsw, tb, out=o, path=path)
    ex.run()
    torch.cuda.synchronize()
    desc = ex.describe()
    ex.close()
    return o.float().cpu().numpy().reshape(-1, w.shape[0]), desc


def tolerance(sums, sa_rows, sw_cols, bias_cols, exact, out):
    p = np.abs(sums.astype(np.float64) * sa_rows.astype(np.float64) *
               sw_cols.astype(np.float64))
    b = 0.0 if bias_cols is None else np.abs(bias_cols.astype(np.float64))
    return 5 * 2.0 ** -24 * (p + b) + UNIT[out] * np.abs(exact) + SUB[out]


def check_scaled(got, sums, exact, sa_rows, sw_cols, bias_cols, out):
    assert np.isfinite(got).all(), "output not written (NaN canary left)"
    tol = tolerance(sums, sa_rows, sw_cols, bias_cols, exact, out)
    err = np.abs(got.astype(np.float64) - exact)
    bad = err > tol
    assert not bad.any(), (
        f"{int(bad.sum())} outputs beyond the bound; worst err {err.max():.3e}")


def tile_of(desc):
    return int(desc.split("tile=")[1].split()[0])


EXACT_SHAPES = [
    (1, 16, 16),
    (5, 7, 32),
    (37, 53, 48),
    (128, 128, 128),
    (129, 257, 272),
    (300, 129, 1040),
    (64, 384, 1024),
    (513, 300, 144),
]


@pytest.mark.parametrize("path", TILES, ids=TILE_IDS)
@pytest.mark.parametrize("m,n,k", EXACT_SHAPES)
def test_integer_sums_exact(m, n, k, path):
    a = codes(11, 7, m, k)
    w = codes(11, 9, n, k)
    ones_m, ones_n = np.ones(m, np.float32), np.ones(n, np.float32)
    got, desc = run_gemm(a, ones_m, w, ones_n, out="f32", path=path)
    assert tile_of(desc) == TILE_SIZE[path], desc
    sums, _ = oracle.w8a8_gemm(a, ones_m, w, ones_n)
    assert np.abs(sums).max() <= 2 ** 24
    assert np.array_equal(got, sums.astype(np.float32)), desc


@pytest.mark.parametrize("path", TILES, ids=TILE_IDS)
def test_extreme_codes_exact(path):
    # -128 * -128 * 1024 = 2^24: the largest sum that float32 holds exactly
    k = 1024
    a = np.full((70, k), -128, np.int8)
    w = np.full((90, k), -128, np.int8)
    w[1::2] = 127
    a[3::5] = 127
    ones_m, ones_n = np.ones(70, np.float32), np.ones(90, np.float32)
    got, _ = run_gemm(a, ones_m, w, ones_n, out="f32", path=path)
    sums, _ = oracle.w8a8_gemm(a, ones_m, w, ones_n)
    assert sums.max() == 2 ** 24
    assert np.array_equal(got, sums.astype(np.float32))


SCALED = [
    (33, 65, 96, "bf16", True),
    (200, 130, 272, "fp16", False),
    (257, 129, 512, "f32", True),
    (130, 300, 1024, "bf16", False),
]


@pytest.mark.parametrize("path", TILES, ids=TILE_IDS)
@pytest.mark.parametrize("m,n,k,out,has_bias", SCALED)
def test_scaled_outputs(m, n, k, out, has_bias, path):
    w8 = synth.GemmWorkload("t", m, n, k, 21 + m, out, has_bias)
    a, sa, w, sw, b = synth.gemm_inputs(w8)
    got, _ = run_gemm(a, sa, w, sw, b, out=out, path=path)
    sums, exact = oracle.w8a8_gemm(a, sa, w, sw, b)
    check_scaled(got, sums, exact, sa[:, None], sw[None, :], None if b is None else b[None, :],
                 out)


@pytest.mark.parametrize("path", TILES, ids=TILE_IDS)
def test_leading_dims(path):
    a = codes(3, 7, 2 * 3 * 7, 64)
    w = codes(3, 9, 40, 64)
    sa = synth.f32(3, 8, synth.UNIFORM, 0.01, 0.08, a.shape[0])
    sw = synth.f32(3, 10, synth.UNIFORM, 1e-4, 1e-3, 40)
    got, _ = run_gemm(a, sa, w, sw, out="f32", lead=(2, 3, 7), path=path)
    sums, exact = oracle.w8a8_gemm(a, sa, w, sw)
    check_scaled(got, sums, exact, sa[:, None], sw[None, :], None, "f32")


@pytest.mark.parametrize("path", TILES, ids=TILE_IDS)
def test_consumes_operator_codes(path):
    """The oracle's own AddRmsNormDynamicQuantV2 codes and scales (bf16
    [300, 1024] rows) feed the GEMM on both sides."""
    wl = synth.WORKLOADS["v2_square"]
    rows, cols = 300, 1024
    x1, x2 = synth.inputs(wl, rows=rows, cols=cols)
    g, b, s1, s2 = synth.params(wl, cols=cols)
    ora = oracle.add_rms_norm_dq_v2(x1, x2, g, b, s1, s2, wl.eps, wl.mask, "int8", "int8",
                                    wl.dtype, want_pre=False)
    a, sa = ora["code1"], ora["scale1"]
    w = codes(wl.seed, 9, 384, cols)
    sw = synth.f32(wl.seed, 10, synth.UNIFORM, 1e-4, 1e-3, 384)
    bias = synth.f32(wl.seed, 11, synth.NORMAL, 0.0, 0.1, 384)
    got, _ = run_gemm(a, sa, w, sw, bias, out="bf16", path=path)
    sums, exact = oracle.w8a8_gemm(a, sa, w, sw, bias)
    check_scaled(got, sums, exact, sa[:, None], sw[None, :], bias[None, :], "bf16")


def sample_positions(m, n, tile, rng, count=6000):
    edges = lambda size: sorted({i for t in range(0, size, tile) for i in (t, t + tile - 1)
                                 if 0 <= i < size} | {0, size - 1, size // 2})
    er, ec = np.array(edges(m)), np.array(edges(n))
    er = er[rng.choice(er.size, min(er.size, 48), replace=False)]
    ec = ec[rng.choice(ec.size, min(ec.size, 48), replace=False)]
    gr, gc = np.meshgrid(er, ec, indexing="ij")
    rows = np.concatenate([gr.ravel(), rng.integers(0, m, count)])
    cols = np.concatenate([gc.ravel(), rng.integers(0, n, count)])
    return rows, cols


@pytest.mark.parametrize("path", [adq.PATH_AUTO] + TILES, ids=["auto"] + TILE_IDS)
@pytest.mark.parametrize("m,n,k,out", [(4100, 3900, 528, "bf16"), (2048, 4096, 1024, "fp16")])
def test_large_ragged_sampled(m, n, k, out, path):
    w8 = synth.GemmWorkload("t", m, n, k, 31, out, True)
    a, sa, w, sw, b = synth.gemm_inputs(w8)
    got, desc = run_gemm(a, sa, w, sw, b, out=out, path=path)
    assert tile_of(desc) in (32, 128, 256), desc
    assert np.isfinite(got).all(), "output not written"
    rows, cols = sample_positions(m, n, tile_of(desc), np.random.default_rng(m))
    sums, exact = oracle.w8a8_gemm_at(a, sa, w, sw, b, rows, cols)
    check_scaled(got[rows, cols], sums, exact, sa[rows], sw[cols], b[cols], out)


def test_full_projection_sampled():
    """16384 x 8192 x 8192, bf16 out: the benchmarked launch."""
    w8 = synth.GEMM_WORKLOADS["w8a8_gemm"]
    a, sa, w, sw, b = synth.gemm_inputs(w8)
    got, desc = run_gemm(a, sa, w, sw, b, out=w8.out_dtype)
    assert tile_of(desc) in (128, 256), desc
    assert np.isfinite(got).all(), "output not written"
    rows, cols = sample_positions(w8.m, w8.n, tile_of(desc), np.random.default_rng(5))
    sums, exact = oracle.w8a8_gemm_at(a, sa, w, sw, b, rows, cols)
    check_scaled(got[rows, cols], sums, exact, sa[rows], sw[cols], None if b is None else b[cols],
                 w8.out_dtype)


def test_full_projection_integer_exact_sampled():
    """Full size with codes in [-45, 45] (|sum| <= 8192 * 45^2 < 2^24) and
    unit scales: sampled outputs equal the exact sums."""
    m, n, k = 16384, 8192, 8192
    a = codes(7, 7, m, k, -45, 45)
    w = codes(7, 9, n, k, -45, 45)
    ones_m, ones_n = np.ones(m, np.float32), np.ones(n, np.float32)
    got, desc = run_gemm(a, ones_m, w, ones_n, out="f32")
    rows, cols = sample_positions(m, n, tile_of(desc), np.random.default_rng(7))
    sums, _ = oracle.w8a8_gemm_at(a, ones_m, w, ones_n, None, rows, cols)
    assert np.array_equal(got[rows, cols], sums.astype(np.float32))


def test_deterministic():
    w8 = synth.GemmWorkload("t", 600, 700, 256, 41, "bf16", True)
    a, sa, w, sw, b = synth.gemm_inputs(w8)
    g1, _ = run_gemm(a, sa, w, sw, b)
    g2, _ = run_gemm(a, sa, w, sw, b)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


def test_paths():
    a = torch.zeros(4, 32, dtype=torch.int8, device="cuda")
    w = torch.zeros(8, 32, dtype=torch.int8, device="cuda")
    sa = torch.ones(4, device="cuda")
    sw = torch.ones(8, device="cuda")
    ex, _ = adq.plan_w8a8_gemm(a, sa, w, sw)
    assert tile_of(ex.describe()) == 32  # few rows: 32-column tiles
    for p in (adq.PATH_ROW, adq.PATH_SPLIT, adq.PATH_GENERIC, 7):
        with pytest.raises(adq.AdqError):
            ex.set_path(p)
    assert ex.set_path(adq.PATH_GEMM_TILE256) == 0 and tile_of(ex.describe()) == 256
    assert ex.set_path(adq.PATH_GEMM_TILE128) == 0 and tile_of(ex.describe()) == 128
    assert ex.set_path(adq.PATH_AUTO) == 0 and tile_of(ex.describe()) == 32
    ex.close()
    a = torch.zeros(300, 32, dtype=torch.int8, device="cuda")
    ex, _ = adq.plan_w8a8_gemm(a, torch.ones(300, device="cuda"), w, sw)
    assert tile_of(ex.describe()) == 128  # more rows, still too few 256-tiles
    ex.close()
    # and the operator's executors refuse the GEMM tile paths
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    ex, _ = adq.plan_add_rms_norm_dynamic_quant_v2(x, x, g)
    for p in TILES:
        with pytest.raises(adq.AdqError):
            ex.set_path(p)
    ex.close()


# ---- few rows (32-column tiles, K split over the wavefronts)

SKINNY_EXACT = [(1, 1, 16), (1, 33, 112), (17, 31, 4096), (32, 64, 8208), (33, 40, 1040),
                (64, 96, 2064), (65, 32, 4096), (100, 70, 528), (128, 33, 4112), (200, 65, 1040)]


@pytest.mark.parametrize("m,n,k", SKINNY_EXACT)
def test_few_rows_integer_sums_exact(m, n, k):
    """Every row block size (32, 64, 128 rows and several blocks), ragged N,
    K past and short of a whole number of 128-byte chunks per wavefront."""
    a = codes(13, 7, m, k)
    w = codes(13, 9, n, k)
    ones_m, ones_n = np.ones(m, np.float32), np.ones(n, np.float32)
    got, desc = run_gemm(a, ones_m, w, ones_n, out="f32", path=adq.PATH_GEMM_TILE32)
    assert tile_of(desc) == 32, desc
    sums, _ = oracle.w8a8_gemm(a, ones_m, w, ones_n)
    assert np.abs(sums).max() <= 2 ** 24
    assert np.array_equal(got, sums.astype(np.float32)), desc


@pytest.mark.parametrize("m", [1, 32, 64, 128, 200])
def test_few_rows_projection_sampled(m):
    """8192 x 8192 projections of decode-sized batches (AUTO), bf16 out with
    bias, against the oracle on sampled outputs (every output written)."""
    w8 = synth.GemmWorkload("t", m, 8192, 8192, 51 + m, "bf16", True)
    a, sa, w, sw, b = synth.gemm_inputs(w8)
    got, desc = run_gemm(a, sa, w, sw, b, out="bf16")
    assert tile_of(desc) == (32 if m <= 128 else 128), desc
    assert np.isfinite(got).all(), "output not written"
    rows, cols = sample_positions(m, 8192, 32, np.random.default_rng(m), count=3000)
    sums, exact = oracle.w8a8_gemm_at(a, sa, w, sw, b, rows, cols)
    check_scaled(got[rows, cols], sums, exact, sa[rows], sw[cols], b[cols], "bf16")
