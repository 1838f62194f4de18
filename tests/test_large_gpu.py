"""Tensors past 4 GiB: every operation addresses them beyond the reach of
32-bit byte offsets.

The row kernel and the GEMM form 64-bit row (tile) bases on the device; the
tiled AddLora kernels use 32-bit offsets, so the library runs a batch whose
y or x reaches 4 GiB as consecutive launch sequences over row ranges below
it.  Inputs are a seeded block of B rows repeated down the whole tensor
(with a ragged tail), which costs no host memory or time at these sizes:
the first B output rows are compared with the oracle under the usual parity
rules, and every other row must equal the block row it repeats, bit for
bit, since each row's result depends only on that row (plus, for the GEMM,
the shared weights; for AddLora, its adapter).  The repetition is checked
on the device in pieces.
"""
import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import oracle
import synth
from gpu_helpers import compare_v2, dev, oracle_v2
from test_lora_gpu import small_ints

pytestmark = pytest.mark.gpu
B = 64
GiB4 = 1 << 32


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def tile_rows(block: torch.Tensor, m: int) -> torch.Tensor:
    """[m, ...] device tensor whose row r is block[r % B]."""
    out = torch.empty((m,) + tuple(block.shape[1:]), dtype=block.dtype, device="cuda")
    q = m // B
    out[:q * B].view((q, B) + tuple(block.shape[1:])).copy_(
        block.unsqueeze(0).expand((q,) + tuple(block.shape)))
    out[q * B:].copy_(block[:m - q * B])
    return out


def assert_periodic(t: torch.Tensor, name: str, piece: int = 512):
    """Every row of t equals row r % B of its first B rows (compared as raw
    bytes, in pieces of `piece` periods)."""
    raw = t.reshape(t.shape[0], -1).view(torch.uint8)
    m = raw.shape[0]
    head = raw[:B]
    q = m // B
    for s in range(0, q, piece):
        e = min(q, s + piece)
        blk = raw[s * B:e * B].view(e - s, B, raw.shape[1])
        if not bool((blk == head.unsqueeze(0)).all()):
            bad = (blk != head.unsqueeze(0)).any(dim=2).nonzero()[0]
            raise AssertionError(f"{name}: row {(s + int(bad[0])) * B + int(bad[1])} differs "
                                 f"from block row {int(bad[1])}")
    if m > q * B:
        assert bool((raw[q * B:] == head[:m - q * B]).all()), f"{name}: tail rows differ"


def test_v2_beyond_4gib():
    """bf16 rows of 8192: x1, x2 and xOut of 8.6 GB (byte offsets past 2^33),
    an INT8 output of 4.3 GB and an INT4 one; 524485 rows (ragged)."""
    n, m = 8192, (1 << 19) + 3 * B + 5
    _announce(f"v2 m={m} n={n} bf16 int8+int4")
    w = synth.Workload("large", "v2", B, n, "bf16", 4242, (True, True), True, 2,
                       outlier_frac=0.01)
    hx1, hx2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    x1 = tile_rows(dev(hx1, "bf16"), m)
    x2 = tile_rows(dev(hx2, "bf16"), m)
    assert x1.numel() * 2 > 2 * GiB4
    y1, y2, sc1, sc2, xo = adq.add_rms_norm_dynamic_quant_v2(
        x1, x2, dev(g, "bf16"), dev(b, "bf16"), dev(s1, "bf16"), dev(s2, "bf16"), 1e-6,
        (True, True), "int8", "int4")
    torch.cuda.synchronize()
    del x1, x2
    assert y1.numel() > GiB4
    ora = oracle_v2(hx1, hx2, g, b, s1, s2, 1e-6, (True, True), ("int8", "int4"), "bf16")
    compare_v2({"x_out": xo[:B], "y1": y1[:B], "y2": y2[:B], "scale1": sc1[:B],
                "scale2": sc2[:B]}, ora, ("int8", "int4"))
    for t, name in ((xo, "x_out"), (y1, "y1"), (y2, "y2"), (sc1.reshape(m, 1), "scale1"),
                    (sc2.reshape(m, 1), "scale2")):
        assert_periodic(t, name)
    del xo, y1, y2
    torch.cuda.empty_cache()


def test_gemm_beyond_4gib():
    """a of 4.3 GB (524389 x 8208) and a float32 output of 4.3 GB (2056
    columns); unit scales, so every output is the exact integer sum."""
    m, k, n = (1 << 19) + B + 37, 8208, 2056
    _announce(f"gemm m={m} n={n} k={k} f32")
    ha = synth.int8_codes(4243, 1, B, k, -127, 127)
    hw = synth.int8_codes(4243, 2, n, k, -127, 127)
    a = tile_rows(torch.from_numpy(ha).cuda(), m)
    assert a.numel() > GiB4
    w = torch.from_numpy(hw).cuda()
    sa = torch.ones(m, dtype=torch.float32, device="cuda")
    sw = torch.ones(n, dtype=torch.float32, device="cuda")
    out = adq.w8a8_gemm(a, sa, w, sw, None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del a
    assert out.numel() * 4 > GiB4
    sums, _ = oracle.w8a8_gemm(ha, np.ones(B, np.float32), hw, np.ones(n, np.float32))
    assert np.array_equal(out[:B].cpu().numpy(), sums.astype(np.float32))
    assert_periodic(out, "out")
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rank,dt,in_place", [(16, "bf16", False), (64, "bf16", True),
                                              (16, "fp16", True)])
def test_lora_beyond_4gib(rank, dt, in_place):
    """y of 4.3 GB (262188 x 8200): two row ranges, 261888 rows (the largest
    multiple of 64 below 4 GiB of y) and 300 (the small-batch sequence).
    Small integers and a power-of-two scale make every fp32 step exact, so
    the block rows equal the oracle's bit for bit; indices include rows
    without an adapter."""
    rows, h1, h2, h3, off, wn, layers, layer = 261888 + 300, 64, 512, 8200, 7680, 5, 2, 1
    _announce(f"lora rows={rows} h3={h3} rank={rank} {dt} in_place={in_place}")
    s = 4244 + rank
    hy = small_ints(s, 13, (B, h3), -8, 8, dt)
    hx = small_ints(s, 12, (B, h1), -2, 2, dt)
    hwa = small_ints(s, 14, (wn, layers, h1, rank), -2, 2, dt)
    hwb = small_ints(s, 15, (wn, layers, rank, h2), -2, 2, dt)
    hidx = synth.int32s(s, 16, -1, wn, B)
    y = tile_rows(dev(hy, dt), rows)
    assert y.numel() * 2 > GiB4
    x = tile_rows(dev(hx, dt), rows)
    idx = tile_rows(torch.from_numpy(hidx).cuda(), rows)
    out = y if in_place else torch.empty_like(y)
    ex, out = adq.plan_add_lora(y, x, dev(hwb, dt), idx, dev(hwa, dt), layer, 0.5, off, out=out)
    desc = ex.describe()
    assert "lora-tiled" in desc and "row_ranges=2" in desc, desc
    ws = torch.full((ex.workspace_size,), 0xA5, dtype=torch.uint8, device="cuda")
    ex.run(ws)
    torch.cuda.synchronize()
    ex.close()
    del x, ws
    if not in_place:
        del y
    ref, _ = oracle.add_lora(hy, hx, hwb, hidx, hwa, layer, 0.5, off, dt)
    got = out[:B].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref), desc
    assert_periodic(out, "out")
    del out
    torch.cuda.empty_cache()


def _gemm_sampled(a, w, out, rows, cols):
    """The GEMM's outputs at (rows[t], cols[t]) against the oracle's exact
    sums (unit scales, float32 output: the sum rounded once on both sides)."""
    sums, _ = oracle.w8a8_gemm_at(a, np.ones(a.shape[0], np.float32), w,
                                  np.ones(w.shape[0], np.float32), None, rows, cols)
    got = out[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    assert np.array_equal(got, sums.astype(np.float32))


def test_gemm_largest_k():
    """k = 131072, the largest accepted (127 * 127 * 2^17 still fits int32):
    rows and columns of +-127 reach the int32 extremes.  Every output of the
    extreme rows and columns, and 2000 random ones, against the oracle."""
    m, n, k = 300, 260, 1 << 17
    _announce(f"gemm m={m} n={n} k={k}")
    a = synth.int8_codes(4245, 1, m, k, -127, 127)
    w = synth.int8_codes(4245, 2, n, k, -127, 127)
    a[0], a[1], w[0], w[1] = 127, -127, 127, -127
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    ex, out = adq.plan_w8a8_gemm(torch.from_numpy(a).cuda(), torch.ones(m, device="cuda"),
                                 torch.from_numpy(w).cuda(), torch.ones(n, device="cuda"), None,
                                 out=out)
    ex.run()
    torch.cuda.synchronize()
    ex.close()
    assert not bool(out.isnan().any())
    assert float(out[0, 0]) == 127 * 127 * k and float(out[1, 0]) == -127 * 127 * k
    rng = np.random.default_rng(4245)
    rows = np.concatenate([np.zeros(n, np.int64), np.ones(n, np.int64), np.arange(m),
                           np.arange(m), rng.integers(0, m, 2000)])
    cols = np.concatenate([np.arange(n), np.arange(n), np.zeros(m, np.int64),
                           np.ones(m, np.int64), rng.integers(0, n, 2000)])
    _gemm_sampled(a, w, out, rows, cols)


def test_gemm_largest_n():
    """n = 2^20 columns, the largest accepted: every output written, the last
    300 columns of every row and 5000 random outputs against the oracle."""
    m, n, k = 40, 1 << 20, 64
    _announce(f"gemm m={m} n={n} k={k}")
    a = synth.int8_codes(4246, 1, m, k, -127, 127)
    w = synth.int8_codes(4246, 2, n, k, -127, 127)
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    ex, out = adq.plan_w8a8_gemm(torch.from_numpy(a).cuda(), torch.ones(m, device="cuda"),
                                 torch.from_numpy(w).cuda(), torch.ones(n, device="cuda"), None,
                                 out=out)
    ex.run()
    torch.cuda.synchronize()
    ex.close()
    assert not bool(out.isnan().any())
    rng = np.random.default_rng(4246)
    rows = np.concatenate([np.repeat(np.arange(m), 300), rng.integers(0, m, 5000)])
    cols = np.concatenate([np.tile(np.arange(n - 300, n), m), rng.integers(0, n, 5000)])
    _gemm_sampled(a, w, out, rows, cols)
