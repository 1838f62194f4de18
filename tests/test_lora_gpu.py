"""Parity of AddLora ("aclnnAddLora", Formulas) on the GPU with the oracle.

Bars:
 - exact: with small-integer x, weights and y and a power-of-two scale every
   fp32 step is exact, so the stored values equal the oracle's bit for bit
   (the structure: grouping, layer, slice, rows without an adapter);
 - realistic data: the kernels sum in fp32 in their own order.  For a slice
   element with exact value v and M = |scale| * sum_r (sum_k |x_k A_kr|) |B_rj|
   (x itself when weightA is absent), recursive fp32 summation of the shrink
   (h1 terms) and the expand (rank terms) errs by at most
   (h1 + rank) * 2^-24 * M; the fused multiply-add into y and the rounding to
   the storage type add 2^-24 |v| and u |v| (u = 2^-8 bf16, 2^-11 fp16) plus
   half the storage type's subnormal spacing:
       |got - v| <= (h1 + rank + 4) 2^-24 M + (2^-24 + u) |v| (1 + 1e-6) + sub
   In bf16 at ranks 32 and above the tiled expand sums on the matrix unit:
   each fp32 z1 value is split exactly into three bf16 pieces, the 3 * rank
   products with weightB are exact, and the bound takes each of their
   additions inside the unit at up to 2^-23 relative (rounding to nearest is
   not assumed there), so 6 * rank stands in for rank.
 - every element outside the slice, and every row without an adapter, equals
   y bit for bit (outputs pre-filled with a canary when out is not y).
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import oracle
import synth
from helpers import from_bits, to_bits

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "fp16": torch.float16}
UNIT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
SUB = {"bf16": 2.0 ** -134, "fp16": 2.0 ** -25}
PATHS = [adq.PATH_AUTO, adq.PATH_GENERIC]
PATH_IDS = ["auto", "generic"]


def dev(bits, dt):
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TD[dt]).to("cuda")


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_lora(y, x, wa, wb, idx, layer, scale, off, dt, path=adq.PATH_AUTO, in_place=False,
             lead=None):
    ty = dev(y, dt)
    if lead is not None:
        ty = ty.reshape(*lead, y.shape[-1])
    tx = dev(x, dt)
    if lead is not None:
        tx = tx.reshape(*lead, x.shape[-1])
    tidx = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to("cuda")
    out = ty if in_place else torch.full_like(ty, float("nan"))
    ex, out = adq.plan_add_lora(ty, tx, dev(wb, dt), tidx, dev(wa, dt), layer, scale, off, out=out,
                                path=path)
    ws = None
    if ex.workspace_size:  # garbage-filled: the grouping pass writes all it reads
        ws = torch.full((ex.workspace_size,), 0xA5, dtype=torch.uint8, device="cuda")
    ex.run(ws)
    torch.cuda.synchronize()
    desc = ex.describe()
    ex.close()
    return bits_of(out).reshape(y.shape), desc


def magnitude(y, x, wa, wb, idx, layer, scale, off, dt, rows=None):
    """M of the bound above for each slice element of the given rows."""
    rows = np.arange(y.shape[0]) if rows is None else np.asarray(rows)
    xv = np.abs(from_bits(x[rows], dt))
    h2 = wb.shape[-1]
    m = np.zeros((rows.size, h2))
    for t, b in enumerate(rows):
        g = idx[b]
        if 0 <= g < wb.shape[0]:
            s1 = xv[t] if wa is None else xv[t] @ np.abs(from_bits(wa[g, layer], dt))
            m[t] = s1 @ np.abs(from_bits(wb[g, layer], dt))
    return m * abs(float(np.float32(scale)))


def expand_terms(rank, dt, desc):
    """Additions the bound charges to one expand sum (see the module notes)."""
    mfma = dt == "bf16" and "mfma-expand" in desc
    return 6 * rank if mfma else rank


def check_slice(got, pre, mag, h1, rank, dt, expand=None):
    gv = from_bits(got, dt)
    expand = rank if expand is None else expand
    tol = (h1 + expand + 4) * 2.0 ** -24 * mag + (2.0 ** -24 + UNIT[dt]) * np.abs(pre) * (1 + 1e-6) \
        + SUB[dt]
    err = np.abs(gv - pre)
    bad = err > tol
    assert not bad.any(), f"{int(bad.sum())} slice values beyond the bound; worst {err.max():.3e}"


def check_outside(got, y, idx, w, off, h2):
    keep = np.ones(y.shape[1], bool)
    keep[off:off + h2] = False
    assert np.array_equal(got[:, keep], y[:, keep]), "columns outside the slice changed"
    none = (idx < 0) | (idx >= w)
    assert np.array_equal(got[none], y[none]), "rows without an adapter changed"


def small_ints(seed, tid, shape, lo, hi, dt):
    v = synth.int8_codes(seed, tid, int(np.prod(shape[:-1])), shape[-1], lo, hi)
    return to_bits(v.astype(np.float64).reshape(shape), dt)


EXACT = [
    # rows, h1, rank, h2, h3, w, layers, layer, off, has_a, dt
    (37, 64, 16, 48, 104, 3, 2, 1, 24, True, "bf16"),
    (700, 64, 16, 48, 104, 3, 2, 1, 24, True, "bf16"),  # above 512 rows: grouping launch
    (700, 64, 16, 48, 104, 100, 2, 1, 24, True, "bf16"),  # 100 adapters
    (8192, 64, 16, 48, 104, 64, 1, 0, 24, True, "bf16"),  # the largest one-workgroup grouping
    (5000, 64, 16, 48, 104, 1, 1, 0, 24, True, "fp16"),   # one adapter
    (4000, 128, 128, 64, 128, 9, 1, 0, 0, True, "bf16"),  # rank 128, 3 slices of h1
    (100, 256, 32, 128, 256, 5, 3, 2, 128, True, "fp16"),
    (17, 16, 16, 64, 64, 2, 1, 0, 0, False, "bf16"),
    (300, 512, 64, 96, 400, 7, 2, 0, 296, True, "bf16"),
    (64, 64, 8, 48, 104, 3, 2, 1, 24, True, "fp16"),     # rank 8 (one padded MFMA block)
    (17, 8, 8, 64, 64, 2, 1, 0, 0, False, "bf16"),       # rank 8 without weightA
    (200, 256, 128, 96, 160, 3, 2, 1, 32, True, "bf16"), # rank 128 (128-k stages)
    (600, 128, 128, 40, 64, 4, 1, 0, 8, True, "bf16"),   # rank 128, grouping launch
    (33, 64, 16, 52, 120, 3, 2, 1, 64, True, "bf16"),   # slice width 4 (mod 8)
    # above 512 rows (grouping launch) at ranks 8 / 16, ragged h1 and slices
    (600, 128, 8, 44, 96, 4, 1, 0, 8, True, "fp16"),    # slice width 4 (mod 8)
    (520, 520, 8, 100, 120, 5, 1, 0, 16, True, "bf16"), # h1 not a multiple of 256
    (1000, 256, 16, 200, 264, 3, 2, 1, 64, True, "bf16"),
    (777, 264, 16, 68, 136, 6, 2, 1, 40, True, "fp16"),
    (50, 64, 64, 96, 160, 3, 1, 0, 32, False, "bf16"),  # matrix-core expand without weightA
    # bf16 at ranks 8 / 16, slices wider than 512 columns
    (800, 64, 16, 640, 1024, 3, 2, 1, 128, True, "bf16"),
    (800, 64, 8, 1100, 1200, 5, 1, 0, 72, True, "bf16"),   # a partial 64-column group
    (40, 16, 16, 2048, 2048, 2, 1, 0, 0, False, "bf16"),   # without weightA
    (600, 128, 128, 64, 128, 2, 1, 0, 0, False, "bf16"),
    # above 8192 rows: the counting and placing launches (3, 2 and 2 workgroups)
    (20000, 64, 16, 48, 104, 5, 2, 1, 24, True, "bf16"),
    (16385, 64, 64, 64, 128, 3, 1, 0, 64, False, "bf16"),
    (8193, 64, 8, 44, 96, 4, 1, 0, 8, True, "fp16"),
    (12000, 64, 16, 48, 104, 1500, 1, 0, 24, True, "fp16"),  # two classes per thread in the layout
    # slices of 257..512 columns: 128-thread expand workgroups (up to 256: 64 threads)
    (700, 64, 16, 400, 480, 3, 2, 1, 64, True, "fp16"),
    (300, 64, 32, 300, 320, 4, 1, 0, 16, True, "fp16"),
    (130, 8, 8, 260, 264, 2, 1, 0, 0, False, "bf16"),
    (37, 64, 16, 48, 100, 3, 2, 1, 20, True, "bf16"),   # y rows not 16-byte aligned: generic
    (5, 30, 5, 7, 13, 2, 2, 1, 3, True, "fp16"),        # generic only (ragged)
]


def tiled_expected(h1, rank, h2, h3, off):
    return (h1 % 8 == 0 and rank in (8, 16, 32, 64, 128) and h2 % 4 == 0 and h3 % 8 == 0
            and off % 8 == 0)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("case", EXACT, ids=[f"{c[0]}x{c[1]}r{c[2]}" for c in EXACT])
def test_exact_integers(case, path):
    rows, h1, rank, h2, h3, w, layers, layer, off, has_a, dt = case
    s = rows + h1
    x = small_ints(s, 12, (rows, h1), -2, 2, dt)
    y = small_ints(s, 13, (rows, h3), -8, 8, dt)
    wa = small_ints(s, 14, (w, layers, h1, rank), -2, 2, dt) if has_a else None
    wb = small_ints(s, 15, (w, layers, rank, h2), -2, 2, dt)
    idx = synth.int32s(s, 16, -1, w, rows)
    got, desc = run_lora(y, x, wa, wb, idx, layer, 0.5, off, dt, path)
    tiled = path == adq.PATH_AUTO and tiled_expected(h1, rank, h2, h3, off)
    assert ("lora-tiled" if tiled else "lora-generic") in desc, desc
    if tiled:
        assert ("count+place" in desc) == (rows > 8192), desc
        # up to 512 rows with weightA, the shrink groups the rows itself
        in_shrink = has_a and rows <= 512
        assert desc.split("kernels=")[1].startswith("shrink") == in_shrink, desc
    ref, _ = oracle.add_lora(y, x, wb, idx, wa, layer, 0.5, off, dt)
    assert np.array_equal(got, ref), desc


# In place (out is y, so rows without an adapter are not listed), above 512
# rows (the grouping launch), ranks 8 / 16, slices wider than 512 columns:
# partial tiles, slices that end inside a 1024-column range, more than 8
# slices of h1, indices outside [0, w), the counting and placing launches.
IN_PLACE = [
    # rows, h1, rank, h2, h3, w, layers, layer, off, dt
    (700, 64, 16, 1100, 1200, 3, 2, 1, 40, "bf16"),
    (2000, 64, 8, 2048, 2304, 5, 1, 0, 256, "fp16"),
    (600, 4096, 16, 1024, 1536, 4, 1, 0, 512, "bf16"),
    (1031, 128, 16, 516, 1032, 7, 2, 1, 8, "fp16"),
    (9000, 64, 16, 600, 608, 2, 1, 0, 0, "bf16"),  # counting and placing launches
    (24576, 1024, 16, 64, 128, 4, 1, 0, 32, "bf16"),  # one slice of 1024 k (8 whole stages)
    (3000, 1000, 8, 96, 104, 5, 2, 1, 8, "fp16"),  # slices ending inside a stage
    (1500, 128, 8, 1028, 1104, 3, 1, 0, 40, "bf16"),
]


@pytest.mark.parametrize("case", IN_PLACE,
                         ids=[f"{c[0]}x{c[1]}r{c[2]}h{c[3]}" for c in IN_PLACE])
def test_exact_integers_in_place(case):
    rows, h1, rank, h2, h3, w, layers, layer, off, dt = case
    s = 31 * rows + h2
    x = small_ints(s, 12, (rows, h1), -2, 2, dt)
    y = small_ints(s, 13, (rows, h3), -8, 8, dt)
    wa = small_ints(s, 14, (w, layers, h1, rank), -2, 2, dt)
    wb = small_ints(s, 15, (w, layers, rank, h2), -2, 2, dt)
    idx = synth.int32s(s, 16, -1, w, rows)
    got, desc = run_lora(y, x, wa, wb, idx, layer, 0.5, off, dt, in_place=True)
    assert "lora-tiled" in desc and "expand" in desc, desc
    ref, _ = oracle.add_lora(y, x, wb, idx, wa, layer, 0.5, off, dt)
    assert np.array_equal(got, ref), desc


@pytest.mark.parametrize("rank", [8, 16, 32, 128])
def test_many_slices_of_h1(rank):
    """Few rows and a long h1: the shrink splits h1 into more than 16 slices,
    so the expand adds the partial sums beyond the first 16 in its second
    loop.  Small integers keep every fp32 step exact: bit-exact."""
    rows, h1, h2, h3, w, layers, layer, off, dt = 40, 8192, 64, 128, 3, 2, 1, 32, "bf16"
    s = 4242 + rank
    x = small_ints(s, 12, (rows, h1), -2, 2, dt)
    y = small_ints(s, 13, (rows, h3), -8, 8, dt)
    wa = small_ints(s, 14, (w, layers, h1, rank), -2, 2, dt)
    wb = small_ints(s, 15, (w, layers, rank, h2), -2, 2, dt)
    idx = synth.int32s(s, 16, -1, w, rows)
    for in_place in (False, True):
        got, desc = run_lora(y, x, wa, wb, idx, layer, 0.5, off, dt, in_place=in_place)
        assert "lora-tiled" in desc and "ksplit=32" in desc, desc
        ref, _ = oracle.add_lora(y, x, wb, idx, wa, layer, 0.5, off, dt)
        assert np.array_equal(got, ref), (in_place, desc)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
@pytest.mark.parametrize("name", ["lora_small", "lora_decode"])
def test_workloads(name, in_place, path):
    wl = synth.LORA_WORKLOADS[name]
    y, x, wa, wb, idx = synth.lora_inputs(wl)
    got, desc = run_lora(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype, path,
                         in_place)
    _, pre = oracle.add_lora(y, x, wb, idx, wa, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    check_outside(got, y, idx, wl.w, wl.y_offset, wl.h2)
    mag = magnitude(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    check_slice(got[:, wl.y_offset:wl.y_offset + wl.h2], pre, mag, wl.h1, wl.rank, wl.dtype,
                expand_terms(wl.rank, wl.dtype, desc))


def oracle_lora_threaded(y, x, wa, wb, idx, layer, scale, off, dt, threads=16):
    """The oracle on every row, cut into contiguous row ranges run on host
    threads at once (its C calls release the GIL), joined in row order: the
    same values as one call over all rows."""
    from concurrent.futures import ThreadPoolExecutor
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    rows = y.shape[0]
    threads = max(1, min(threads, cores, rows))
    cuts = [rows * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(threads) as pool:
        parts = list(pool.map(
            lambda i: oracle.add_lora(y, x, wb, idx, wa, layer, scale, off, dt,
                                      rows=np.arange(cuts[i], cuts[i + 1])), range(threads)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def magnitude_all(x, wa, wb, idx, layer, scale, dt):
    """M of the bound for every row, one adapter at a time as matrix
    products (the same sums as magnitude(), in another order; M only scales
    the tolerance)."""
    h2 = wb.shape[-1]
    m = np.zeros((x.shape[0], h2))
    for g in range(wb.shape[0]):
        sel = np.flatnonzero(idx == g)
        if sel.size:
            s1 = np.abs(from_bits(x[sel], dt)) @ np.abs(from_bits(wa[g, layer], dt))
            m[sel] = s1 @ np.abs(from_bits(wb[g, layer], dt))
    return m * abs(float(np.float32(scale)))


def test_prefill_full_size_every_row():
    """4096 rows x 4096 -> 16 -> 4096 into a 12288-wide y, in place (the
    benchmarked launch): every row's slice against the oracle element by
    element under the bound, every row's columns outside the slice bit for
    bit."""
    wl = synth.LORA_WORKLOADS["lora_prefill"]
    y, x, wa, wb, idx = synth.lora_inputs(wl)
    got, desc = run_lora(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype,
                         in_place=True)
    assert "lora-tiled" in desc, desc
    check_outside(got, y, idx, wl.w, wl.y_offset, wl.h2)
    ref, pre = oracle_lora_threaded(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    assert pre.shape == (wl.rows, wl.h2)
    mag = magnitude_all(x, wa, wb, idx, wl.layer, wl.scale, wl.dtype)
    check_slice(got[:, wl.y_offset:wl.y_offset + wl.h2], pre, mag, wl.h1, wl.rank, wl.dtype,
                expand_terms(wl.rank, wl.dtype, desc))


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("rank", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("rows,h2,h3,off", [(300, 384, 1024, 128), (700, 2560, 4096, 1024)],
                         ids=["one_chunk", "three_chunks"])
def test_ranks_realistic(rows, h2, h3, off, rank, dt):
    """Normal data at every tiled rank, against the bound: 300 rows
    (grouping inside the shrink) and 700 rows (grouping launch), a slice of
    384 columns or 2560; indices include values outside [0, w)."""
    wl = dataclasses.replace(synth.LORA_WORKLOADS["lora_small"], name=f"lora_r{rank}",
                             rows=rows, rank=rank, h2=h2, h3=h3, y_offset=off, dtype=dt)
    y, x, wa, wb, idx = synth.lora_inputs(wl)
    got, desc = run_lora(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, dt)
    assert "lora-tiled" in desc, desc
    _, pre = oracle.add_lora(y, x, wb, idx, wa, wl.layer, wl.scale, wl.y_offset, dt)
    check_outside(got, y, idx, wl.w, wl.y_offset, wl.h2)
    mag = magnitude(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, dt)
    check_slice(got[:, off:off + h2], pre, mag, wl.h1, rank, dt, expand_terms(rank, dt, desc))


@pytest.mark.parametrize("pattern", ["one_adapter", "distinct", "none", "single_row",
                                     "many_adapters"])
def test_grouping_patterns(pattern):
    rows, h1, rank, h2, h3, layers, dt = 96, 128, 16, 64, 128, 2, "bf16"
    w = {"many_adapters": 2048, "distinct": 96}.get(pattern, 4)
    if pattern == "single_row":
        rows = 1
    s = 77
    x = small_ints(s, 12, (rows, h1), -2, 2, dt)
    y = small_ints(s, 13, (rows, h3), -8, 8, dt)
    wa = small_ints(s, 14, (w, layers, h1, rank), -2, 2, dt)
    wb = small_ints(s, 15, (w, layers, rank, h2), -2, 2, dt)
    idx = {
        "one_adapter": np.full(rows, 2, np.int32),
        "distinct": np.random.default_rng(1).permutation(rows).astype(np.int32),
        "none": np.full(rows, -5, np.int32),
        "single_row": np.array([1], np.int32),
        "many_adapters": synth.int32s(s, 16, 0, w - 1, rows),
    }[pattern]
    for in_place in (False, True):
        got, desc = run_lora(y, x, wa, wb, idx, 1, 0.25, 32, dt, in_place=in_place)
        ref, _ = oracle.add_lora(y, x, wb, idx, wa, 1, 0.25, 32, dt)
        assert np.array_equal(got, ref), (pattern, in_place, desc)


def test_leading_dims_and_determinism():
    wl = synth.LORA_WORKLOADS["lora_small"]
    y, x, wa, wb, idx = synth.lora_inputs(wl)
    lead = (3, 100)
    g1, _ = run_lora(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype, lead=lead)
    g2, _ = run_lora(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    assert np.array_equal(g1, g2)
    g3, _ = run_lora(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    assert np.array_equal(g2, g3)


def test_paths():
    wl = synth.LORA_WORKLOADS["lora_small"]
    y, x, wa, wb, idx = synth.lora_inputs(wl, rows=8)
    ty, tx = dev(y, "bf16"), dev(x, "bf16")
    ex, _ = adq.plan_add_lora(ty, tx, dev(wb, "bf16"), torch.from_numpy(idx).cuda(),
                              dev(wa, "bf16"), wl.layer, wl.scale, wl.y_offset)
    assert "lora-tiled" in ex.describe()
    for p in (adq.PATH_ROW, adq.PATH_SPLIT, adq.PATH_GEMM_TILE128):
        with pytest.raises(adq.AdqError):
            ex.set_path(p)
    assert ex.workspace_size > 0
    assert ex.set_path(adq.PATH_GENERIC) == 0
    assert "lora-generic" in ex.describe()
    assert ex.set_path(adq.PATH_AUTO) > 0
    assert "lora-tiled" in ex.describe()
    ex.close()


@pytest.mark.parametrize("rank,rows,slices", [(16, 4096, 6), (64, 4096, 6), (128, 4096, 3),
                                               (16, 64, 16), (128, 64, 16)])
def test_slices_of_h1(rank, rows, slices):
    """Slices of h1 per tile planned for the prefill and decode shapes (h1
    4096, 8 adapters) on a 256-CU device: 1.5 shrink workgroups per CU, 0.75 at
    rank 128, over rows / 64 + 8 estimated tiles, every slice at least 256 k
    (so at most 16); fewer when the shrink instance holds fewer per CU."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("slice counts stated for 256 CUs")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    y = torch.empty(rows, 12288, **bf)
    x = torch.empty(rows, 4096, **bf)
    wb = torch.empty(8, 32, rank, 4096, **bf)
    wa = torch.empty(8, 32, 4096, rank, **bf)
    idx = torch.zeros(rows, dtype=torch.int32, device="cuda")
    ex, _ = adq.plan_add_lora(y, x, wb, idx, wa, 7, 0.5, 4096, out=y)
    desc = ex.describe()
    ex.close()
    assert f" ksplit={slices} " in desc, desc


@pytest.mark.parametrize("h2,kind", [((1 << 24) - 8, "lora-tiled"), (1 << 24, "lora-generic")])
def test_offset_limits_select_the_kernel(h2, kind):
    """The tiled kernels address weightB[g, layer] with 32-bit byte offsets
    (y and x are taken in row ranges below 4 GiB): a rank-128 weightB slice
    of 2^32 bytes (2^24 columns) is planned
    on the generic kernel, one just below on the tiled kernels.  Planning
    only (tensors left uninitialised)."""
    rank = 128
    y = torch.empty((2, h2), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((2, 64), dtype=torch.bfloat16, device="cuda")
    wa = torch.empty((1, 1, 64, rank), dtype=torch.bfloat16, device="cuda")
    wb = torch.empty((1, 1, rank, h2), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(2, dtype=torch.int32, device="cuda")
    ex, _ = adq.plan_add_lora(y, x, wb, idx, wa, 0, 0.5, 0, out=y)
    desc = ex.describe()
    ex.close()
    del y, x, wa, wb
    torch.cuda.empty_cache()
    assert kind in desc, desc
