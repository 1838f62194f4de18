"""The AddRmsNormDynamicQuantV2 entry point that allocates nothing
(adq_add_rms_norm_dynamic_quant_v2_no_alloc), through the C-ABI, against the
entry point with a caller's workspace: the same executor plans run both
ways must give the same bits.  Two calls in a row, the second on a smaller
input, on each path whose kernels use scratch memory (the split-row path's
one-, two- and three-launch forms) and on one that uses none (the row
kernel); plans needing more than the static buffer are refused; a captured
call replays like an eager one."""
import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import synth
from gpu_helpers import compare_v2, dev, oracle_v2

pytestmark = pytest.mark.gpu
SCRATCH_BYTES = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield


def _inputs(m, n, dtype, seed):
    w = synth.Workload("noalloc", "v2", m, n, dtype, seed, None, True, 2)
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    return x1, x2, g, b, s1, s2


def _plan(host, dtype, path, launches):
    x1, x2, g, b, s1, s2 = host
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
        dev(x1, dtype), dev(x2, dtype), dev(g, dtype), dev(b, dtype), dev(s1, dtype),
        dev(s2, dtype), 1e-6, None, "int8", "int4", path=path)
    if launches:
        ex.set_split(0, launches)
    return ex, outs


def _both_ways(host, dtype, path, launches):
    """Outputs of the no-alloc call and of the workspace call of one plan."""
    ex, outs = _plan(host, dtype, path, launches)
    ref_ex, ref = _plan(host, dtype, path, launches)
    assert ex.describe() == ref_ex.describe()
    assert ex.workspace_size <= SCRATCH_BYTES
    ex.run_no_alloc()
    ws = (torch.empty(ref_ex.workspace_size, dtype=torch.uint8, device="cuda")
          if ref_ex.workspace_size else None)
    ref_ex.run(ws)
    torch.cuda.synchronize()
    desc = ex.describe()
    ex.close()
    ref_ex.close()
    return outs, ref, desc


CASES = [  # (path, launches, larger shape, smaller shape, dtype)
    (adq.PATH_AUTO, 0, (32, 16384), (5, 16384), "bf16"),      # split, one launch
    (adq.PATH_SPLIT, 2, (48, 8192), (7, 4096), "fp16"),        # split, two launches
    (adq.PATH_SPLIT, 3, (40, 32768), (3, 16384), "bf16"),     # split, three launches
    (adq.PATH_AUTO, 0, (3, 65536), (1, 40008), "fp16"),        # long rows
    (adq.PATH_ROW, 0, (300, 4096), (17, 1024), "bf16"),        # row kernel: no scratch
]


@pytest.mark.parametrize("path,launches,big,small,dtype", CASES)
def test_no_alloc_matches_workspace_call_twice(path, launches, big, small, dtype):
    print(f"\n[case] no_alloc path={path} launches={launches} {big} then {small} {dtype}",
          flush=True)
    for k, (m, n) in enumerate((big, small)):
        host = _inputs(m, n, dtype, seed=700 + 10 * k + m)
        outs, ref, desc = _both_ways(host, dtype, path, launches)
        if path == adq.PATH_AUTO and n >= 16384:
            assert "path=split" in desc, desc
        for key in ("x_out", "y1", "y2", "scale1", "scale2"):
            assert torch.equal(outs[key], ref[key]), (key, m, n)
        ora = oracle_v2(*host, 1e-6, None, ("int8", "int4"), dtype)
        compare_v2(outs, ora, ("int8", "int4"))


def test_no_alloc_refuses_plans_beyond_the_buffer():
    """100000 rows of 8 columns on the three-launch split form need 1.2 MB of
    partial results: more than the 1 MiB buffer."""
    host = _inputs(100000, 8, "bf16", seed=9)
    ex, _ = _plan(host, "bf16", adq.PATH_SPLIT, 3)
    assert ex.workspace_size > SCRATCH_BYTES
    with pytest.raises(adq.AdqError) as e:
        ex.run_no_alloc()
    assert e.value.status == adq.ERR_WORKSPACE
    ex.close()


def test_no_alloc_rejects_other_executors():
    x = dev(_inputs(4, 1024, "fp16", 10)[0], "fp16")
    g = dev(_inputs(4, 1024, "fp16", 10)[2], "fp16")
    ex, _ = adq.plan_rms_norm_dynamic_quant(x, g, None, None, 1e-6, "int8")
    status = adq.lib.adq_add_rms_norm_dynamic_quant_v2_no_alloc(ex.handle, None)
    assert status == adq.ERR_PARAM_INVALID
    assert adq.lib.adq_add_rms_norm_dynamic_quant_v2_no_alloc(None, None) == adq.ERR_NULLPTR
    ex.close()


def test_no_alloc_call_captured_and_replayed():
    """A no-alloc call captured into a graph (the split-row path then runs its
    plain-launch form on the static buffer), replayed with new inputs written
    in place, equals an eager no-alloc call every time."""
    m, n, dtype = 32, 16384, "bf16"
    host = _inputs(m, n, dtype, seed=11)
    ex, outs = _plan(host, dtype, adq.PATH_AUTO, 0)
    ref_ex, ref = _plan(host, dtype, adq.PATH_AUTO, 0)
    assert "path=split" in ex.describe()
    x1, x2 = ex._keep[1], ex._keep[2]
    rx1, rx2 = ref_ex._keep[1], ref_ex._keep[2]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ex.run_no_alloc(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ex.run_no_alloc()
    torch.cuda.synchronize()
    w = synth.Workload("noalloc", "v2", m, n, dtype, 11, None, True, 2)
    for rep in range(3):
        n1, n2 = synth.inputs(w, seed=800 + rep)
        for t, r, a in ((x1, rx1, n1), (x2, rx2, n2)):
            t.copy_(dev(a, dtype))
            r.copy_(dev(a, dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_ex.run_no_alloc()
        torch.cuda.synchronize()
        for key in ("x_out", "y1", "y2", "scale1", "scale2"):
            assert torch.equal(outs[key], ref[key]), (key, rep)
    ex.close()
    ref_ex.close()
