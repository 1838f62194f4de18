"""GPU tests of the split-row path (several workgroups per row exchanging
partial sums and maxima through the workspace), against the oracle."""
import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import synth
from gpu_helpers import (check_no_timeout, compare_v2, dev, host, host_bits, oracle_v2, run_rms,
                         run_v2, workspace)
from gpu_helpers import compare_rms
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield


def _inputs(m, n, dtype, seed, n_smooth=2):
    w = synth.Workload("split", "v2", m, n, dtype, seed, None, True, n_smooth)
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    return x1, x2, g, b, s1, s2


SPLIT_SHAPES = [(1, 2048), (3, 4096), (32, 16384), (7, 16392), (5, 20000), (2, 65536),
                (64, 8192), (257, 32768), (9, 8), (130, 1024)]


@pytest.mark.parametrize("m,n", SPLIT_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_split_path_parity(m, n, dtype):
    print(f"\n[case] split {m}x{n} {dtype}", flush=True)
    y_types = ("int8", "int4")
    x1, x2, g, b, s1, s2 = _inputs(m, n, dtype, seed=300 + m + n)
    outs, desc = run_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True), y_types, dtype,
                        path=adq.PATH_SPLIT)
    assert "path=split" in desc, desc
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True), y_types, dtype)
    compare_v2(outs, ora, y_types)


@pytest.mark.parametrize("fill", [None, 0x00, 0xFF, 0xA5])
def test_split_workspace_contents_do_not_matter(fill):
    x1, x2, g, b, s1, s2 = _inputs(32, 16384, "bf16", seed=5)
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16")
    outs, desc = run_v2(x1, x2, g, b, s1, s2, 1e-6, None, ("int8", "int8"), "bf16",
                        path=adq.PATH_SPLIT, ws_fill=fill)
    compare_v2(outs, ora, ("int8", "int8"))


def test_split_reused_workspace_and_determinism():
    """Back-to-back launches on one workspace (which then holds the previous
    launch's slots) give bitwise-identical results; new inputs in the same
    buffers give the new results."""
    x1, x2, g, b, s1, s2 = _inputs(16, 8192, "bf16", seed=6)
    d1, d2 = dev(x1, "bf16"), dev(x2, "bf16")
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
        d1, d2, dev(g, "bf16"), dev(b, "bf16"), dev(s1, "bf16"), dev(s2, "bf16"), 1e-6, None,
        path=adq.PATH_SPLIT)
    ws = workspace(ex)
    ex.run(ws)
    torch.cuda.synchronize()
    check_no_timeout(ex, ws)
    first = {k: v.clone() for k, v in outs.items() if v is not None}
    for _ in range(5):
        ex.run(ws)
    torch.cuda.synchronize()
    check_no_timeout(ex, ws)
    for k, v in first.items():
        assert torch.equal(outs[k], v), k
    y1, y2, _, _, _, _ = _inputs(16, 8192, "bf16", seed=7)
    d1.copy_(dev(y1, "bf16"))
    d2.copy_(dev(y2, "bf16"))
    ex.run(ws)
    torch.cuda.synchronize()
    check_no_timeout(ex, ws)
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


@pytest.mark.parametrize("mask,has1,has2", [((False, True), False, True), ((True, False), True, False),
                                            (None, False, False), ((True, True), False, False)])
def test_split_output_options(mask, has1, has2):
    x1, x2, g, b, s1, s2 = _inputs(6, 4096, "bf16", seed=10)
    s1 = s1 if has1 else None
    s2 = s2 if has2 else None
    outs, _ = run_v2(x1, x2, g, b, s1, s2, 1e-6, mask, ("int4", "int8"), "bf16",
                     path=adq.PATH_SPLIT)
    ora = oracle_v2(x1, x2, g, b, s1, s2, 1e-6, mask, ("int4", "int8"), "bf16")
    compare_v2(outs, ora, ("int4", "int8"))


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
