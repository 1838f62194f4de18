"""GPU tests of the split-row path: S workgroups per row, each on a chunk,
handing the per-chunk partial sums of squares and maxima over through the
workspace -- in one launch (tagged slots, bounded waits, missing partial
results computed locally) or in two or three plain launches per batch of
rows.  Compared with the oracle under the parity rules, through the C-ABI."""
import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import oracle
import synth
from gpu_helpers import compare_rms, compare_v2, dev, oracle_v2, run_rms, run_v2, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(m, n, dtype, seed, n_smooth=2):
    w = synth.Workload("split", "v2", m, n, dtype, seed, None, True, n_smooth)
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    return x1, x2, g, b, s1, s2


def _run_split(x1, x2, g, b, s1, s2, mask, y_types, dtype, splits=0, launches=0, ws_fill=None,
               eps=1e-6, wait_us=-1, spread=False):
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
        dev(x1, dtype), dev(x2, dtype), dev(g, dtype), dev(b, dtype), dev(s1, dtype),
        dev(s2, dtype), eps, mask, y_types[0], y_types[1], path=adq.PATH_SPLIT)
    if splits or launches or wait_us >= 0 or spread:
        ex.set_split(splits, launches, wait_us, spread)
    ws = workspace(ex, ws_fill)
    ex.run(ws)
    torch.cuda.synchronize()
    desc = ex.describe()
    ex.close()
    return outs, desc


SPLIT_SHAPES = [(1, 2048), (3, 4096), (32, 16384), (7, 16392), (5, 20000), (2, 65536),
                (64, 8192), (257, 32768), (9, 8), (130, 1024), (1, 262144), (3, 40008)]


@pytest.mark.parametrize("launches", [1, 2, 3])
@pytest.mark.parametrize("m,n", SPLIT_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_split_path_parity(m, n, dtype, launches):
    _announce(f"split {m}x{n} {dtype} launches={launches}")
    y_types = ("int8", "int4")
    x1, x2, g, b, s1, s2 = _inputs(m, n, dtype, seed=300 + m + n)
    outs, desc = _run_split(x1, x2, g, b, s1, s2, (True, True), y_types, dtype,
                            launches=launches)
    assert "path=split" in desc and f"launches={launches}" in desc, desc
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True), y_types, dtype)
    compare_v2(outs, ora, y_types)


@pytest.mark.parametrize("splits", [2, 3, 8, 64])
def test_split_counts(splits):
    """Explicit chunk counts on 9 x 32768 (4096 vectors per row): chunks of
    2048, 1408 (ragged last chunk), 512 and 64 vectors."""
    _announce(f"split 9x32768 bf16 splits={splits}")
    x1, x2, g, b, s1, s2 = _inputs(9, 32768, "bf16", seed=31)
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16")
    for launches in (1, 2, 3):
        outs, desc = _run_split(x1, x2, g, b, s1, s2, None, ("int8", "int8"), "bf16",
                                splits=splits, launches=launches)
        assert f"splits={splits} " in desc, desc
        compare_v2(outs, ora, ("int8", "int8"))


def test_split_count_that_does_not_fit_is_rejected():
    x1, x2, g, b, s1, s2 = _inputs(2, 32768, "bf16", seed=32)
    ex, _ = adq.plan_add_rms_norm_dynamic_quant_v2(
        dev(x1, "bf16"), dev(x2, "bf16"), dev(g, "bf16"), None, None, None, 1e-6, None)
    before = ex.describe()
    # 1 chunk > 2048 vectors; no 4-launch form; negative count; > 64 chunks in one launch
    for splits, launches in ((1, 0), (0, 4), (-1, 2), (65, 1)):
        with pytest.raises(adq.AdqError) as e:
            ex.set_split(splits, launches)
        assert e.value.status == adq.ERR_PARAM_INVALID
        assert ex.describe() == before
    ex.close()


@pytest.mark.parametrize("m,n,dtype", [(40, 12288, "fp16"), (32, 16384, "bf16"),
                                         (3, 40008, "bf16")])
def test_launch_forms_agree_bit_for_bit(m, n, dtype):
    """For one chunk count every form quantizes the same fp32 values with the
    same scale, so every output is the same bits: the three launch forms, the
    one-launch form with no waiting (partial results of chunks whose slots are
    not there at the first look are computed by the waiting workgroup) and
    with a row's chunks on different XCDs."""
    _announce(f"forms {m}x{n} {dtype}")
    x1, x2, g, b, s1, s2 = _inputs(m, n, dtype, seed=33)
    ref, desc = _run_split(x1, x2, g, b, s1, s2, None, ("int8", "int4"), dtype, launches=3)
    splits = int(desc.split("splits=")[1].split()[0])
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int4"), dtype)
    compare_v2(ref, ora, ("int8", "int4"))
    for launches, wait_us, spread in ((2, -1, False), (1, -1, False), (1, 0, False),
                                      (1, -1, True), (1, 0, True)):
        got, d = _run_split(x1, x2, g, b, s1, s2, None, ("int8", "int4"), dtype,
                            splits=splits, launches=launches, wait_us=wait_us, spread=spread)
        assert f"launches={launches} " in d and f"spread={int(spread)} " in d, d
        for k in ("x_out", "y1", "y2", "scale1", "scale2"):
            assert torch.equal(ref[k], got[k]), (k, launches, wait_us, spread)


def test_split_batches_of_rows():
    """300 rows of 65536 bf16 columns: x1 and x2 take 256 KiB per row, so the
    rows run as a batch of 256 and a batch of 44 (each batch's launches
    before the next batch's), sharing one workspace."""
    m, n = 300, 65536
    _announce(f"split batches {m}x{n}")
    x1, x2, g, b, s1, s2 = _inputs(m, n, "bf16", seed=34)
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16")
    for launches in (2, 3):
        outs, desc = _run_split(x1, x2, g, b, s1, s2, None, ("int8", "int8"), "bf16",
                                launches=launches)
        assert "batch_rows=256 " in desc, desc
        compare_v2(outs, ora, ("int8", "int8"))
    # the one-launch form in batches of rows whose workgroups fit on the chip
    outs, desc = _run_split(x1, x2, g, b, s1, s2, None, ("int8", "int8"), "bf16", launches=1)
    assert int(desc.split("batch_rows=")[1].split()[0]) < m, desc
    compare_v2(outs, ora, ("int8", "int8"))


@pytest.mark.parametrize("fill", [None, 0x00, 0xFF, 0xA5])
def test_split_workspace_contents_do_not_matter(fill):
    x1, x2, g, b, s1, s2 = _inputs(32, 16384, "bf16", seed=5)
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16")
    for launches in (1, 2, 3):
        outs, desc = _run_split(x1, x2, g, b, s1, s2, None, ("int8", "int8"), "bf16",
                                launches=launches, ws_fill=fill)
        compare_v2(outs, ora, ("int8", "int8"))


def test_split_reused_workspace_and_determinism():
    """Back-to-back launches on one workspace (which then holds the previous
    launch's partial results) give bitwise-identical results; new inputs in
    the same buffers give the new results."""
    x1, x2, g, b, s1, s2 = _inputs(16, 8192, "bf16", seed=6)
    d1, d2 = dev(x1, "bf16"), dev(x2, "bf16")
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
        d1, d2, dev(g, "bf16"), dev(b, "bf16"), dev(s1, "bf16"), dev(s2, "bf16"), 1e-6, None,
        path=adq.PATH_SPLIT)
    ws = workspace(ex)
    ex.run(ws)
    torch.cuda.synchronize()
    first = {k: v.clone() for k, v in outs.items() if v is not None}
    for _ in range(5):
        ex.run(ws)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(outs[k], v), k
    y1, y2, _, _, _, _ = _inputs(16, 8192, "bf16", seed=7)
    d1.copy_(dev(y1, "bf16"))
    d2.copy_(dev(y2, "bf16"))
    ex.run(ws)
    torch.cuda.synchronize()
    ora = oracle_v2(y1, y2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16")
    compare_v2(outs, ora, ("int8", "int8"))
    ex.close()


def test_split_and_row_paths_agree_on_xout():
    x1, x2, g, b, s1, s2 = _inputs(48, 8192, "fp16", seed=8)
    a, _ = run_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "fp16",
                  path=adq.PATH_SPLIT)
    r, _ = run_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "fp16",
                  path=adq.PATH_ROW)
    assert torch.equal(a["x_out"], r["x_out"])


@pytest.mark.parametrize("y_type", ["int8", "int4"])
def test_split_rms_norm_dq(y_type):
    w = synth.Workload("rms", "rmsnorm", 12, 16384, "fp16", 9, None, True, 1)
    x, _ = synth.inputs(w)
    g, b, s1, _ = synth.params(w)
    outs, desc = run_rms(x, g, b, s1, 1e-6, y_type, "fp16", path=adq.PATH_SPLIT)
    assert "path=split" in desc
    compare_rms(outs, oracle.rms_norm_dq(x, g, b, s1, 1e-6, y_type, "fp16"), y_type)
    for launches in (1, 2, 3):
        ex, o = adq.plan_rms_norm_dynamic_quant(dev(x, "fp16"), dev(g, "fp16"), dev(b, "fp16"),
                                                dev(s1, "fp16"), 1e-6, y_type)
        ex.set_split(0, launches)
        ex.run(workspace(ex))
        torch.cuda.synchronize()
        ex.close()
        for k in ("y", "scale"):
            assert torch.equal(o[k], outs[k]), (k, launches)


@pytest.mark.parametrize("mask,has1,has2", [((False, True), False, True), ((True, False), True, False),
                                            (None, False, False), ((True, True), False, False)])
def test_split_output_options(mask, has1, has2):
    x1, x2, g, b, s1, s2 = _inputs(6, 4096, "bf16", seed=10)
    s1 = s1 if has1 else None
    s2 = s2 if has2 else None
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, mask, ("int4", "int8"), "bf16")
    for launches in (1, 2, 3):
        outs, _ = _run_split(x1, x2, g, b, s1, s2, mask, ("int4", "int8"), "bf16",
                             launches=launches)
        compare_v2(outs, ora, ("int4", "int8"))


@pytest.mark.parametrize("launches", [1, 2, 3])
def test_split_degenerate_rows(launches):
    """gamma = beta = 0 (row maximum 0: scale 0, codes 0), and x = 0 with
    epsilon = 0 (0/0 in the norm, read as row maximum 0), on the split path."""
    m, n = 3, 4096
    x1, x2, g, b, s1, s2 = _inputs(m, n, "bf16", seed=12)
    zero = np.zeros(n, np.uint16)
    outs, _ = _run_split(x1, x2, zero, zero, None, None, (True, True), ("int8", "int8"),
                         "bf16", launches=launches)
    for k in (1, 2):
        assert torch.all(outs[f"scale{k}"] == 0) and torch.all(outs[f"y{k}"] == 0)
    zx = np.zeros((m, n), np.uint16)
    outs, _ = _run_split(zx, zx, g, zero, None, None, None, ("int8", "int8"), "bf16",
                         launches=launches, eps=0.0)
    assert torch.all(outs["scale1"] == 0) and torch.all(outs["y1"] == 0)


def test_split_workspace_errors():
    x1, x2, g, b, s1, s2 = _inputs(4, 4096, "bf16", seed=11)
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
        dev(x1, "bf16"), dev(x2, "bf16"), dev(g, "bf16"), None, None, None, 1e-6, None,
        path=adq.PATH_SPLIT)
    assert ex.workspace_size > 0
    small = torch.empty(ex.workspace_size - 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(adq.AdqError) as e:
        ex.run(small)
    assert e.value.status == adq.ERR_WORKSPACE
    with pytest.raises(adq.AdqError) as e:
        ex.run(None)
    assert e.value.status == adq.ERR_WORKSPACE
    big = torch.empty(ex.workspace_size + 16, dtype=torch.uint8, device="cuda")
    status = adq.lib.adq_add_rms_norm_dynamic_quant_v2(big.data_ptr() + 4, ex.workspace_size,
                                                       ex.handle, None)
    assert status == adq.ERR_WORKSPACE
    ex.close()


def test_one_shot_helper_on_side_stream_keeps_workspace():
    """The one-shot helper allocates the workspace and the outputs on torch's
    current stream and launches on a side stream; they are marked as used
    there, so memory allocated on the current stream right after the call
    (and filled before the side stream ends) does not take them over."""
    m, n = 32, 16384
    x1, x2, g, b, s1, s2 = _inputs(m, n, "bf16", seed=13)
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16")
    args = [dev(a, "bf16") for a in (x1, x2, g, b, s1, s2)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        # a long kernel first on the side stream, so the operator runs late
        spin = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(side):
            spin.fill_(1)
        y1, y2, sc1, sc2, xo = adq.add_rms_norm_dynamic_quant_v2(
            *args, 1e-6, None, path=adq.PATH_SPLIT, stream=side)
        junk = [torch.full((1 << 16,), 0x7F, dtype=torch.uint8, device="cuda")
                for _ in range(8)]
        side.synchronize()
        torch.cuda.synchronize()
        outs = {"x_out": xo, "y1": y1, "y2": y2, "scale1": sc1, "scale2": sc2}
        compare_v2(outs, ora, ("int8", "int8"))
        del junk, spin
