"""Phase 2 under HIP graph capture.

The run calls allocate nothing and never synchronize, so a caller can
capture them into a graph (torch.cuda.graph here) and replay it.  Each test
captures one run, then replays it several times with new input values
written in place between replays (eager work and synchronizations in
between), and checks every replay bit for bit against an eager call on the
same inputs.
"""
import numpy as np
import pytest
import torch

import int4_dynamic_quantization_amd as adq
import synth
from gpu_helpers import dev, host_bits
from test_lora_gpu import small_ints

pytestmark = pytest.mark.gpu
REPLAYS = 3


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().copy()


@pytest.mark.parametrize("m,n,dtype,y_types", [(96, 4096, "bf16", ("int8", "int4")),
                                               (257, 1000, "fp16", ("int8", "int8"))])
def test_v2_replays_match_eager(m, n, dtype, y_types):
    w = synth.Workload("graph", "v2", m, n, dtype, 77, (True, True), True, 2)
    g, b, s1, s2 = (dev(p, dtype) for p in synth.params(w))
    x1, x2 = (dev(a, dtype) for a in synth.inputs(w))
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True),
                                                      y_types[0], y_types[1])
    assert "path=split" not in ex.describe()
    graph = capture(lambda: ex.run(None))
    previous = None
    for rep in range(REPLAYS):
        n1, n2 = synth.inputs(w, seed=500 + rep)
        x1.copy_(dev(n1, dtype))
        x2.copy_(dev(n2, dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(outs[k]) for k in ("x_out", "y1", "y2", "scale1", "scale2")]
        ref = adq.add_rms_norm_dynamic_quant_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True),
                                                y_types[0], y_types[1])
        torch.cuda.synchronize()
        want = [bits(t) for t in (ref[4], ref[0], ref[1], ref[2], ref[3])]
        for a_, b_ in zip(got, want):
            assert np.array_equal(a_, b_), f"replay {rep} differs from the eager call"
        assert previous is None or not np.array_equal(got[0], previous), "replay saw stale inputs"
        previous = got[0]
    ex.close()


@pytest.mark.parametrize("launches", [1, 2, 3])
def test_v2_split_path_replays_match_eager(launches):
    """The split-row path (decode shape 32 x 16384: several workgroups per
    row, partial results handed over through the workspace); the eager
    reference runs the same plan.  With the one-launch form the captured call
    runs the plain-launch form (the capture would freeze the one-launch
    form's tag) while the eager reference runs the one-launch form: every
    replay must still equal it bit for bit."""
    m, n, dtype, y_types = 32, 16384, "bf16", ("int8", "int8")
    w = synth.Workload("graph", "v2", m, n, dtype, 81, (True, True), True, 2)
    g, b, s1, s2 = (dev(p, dtype) for p in synth.params(w))
    x1, x2 = (dev(a, dtype) for a in synth.inputs(w))
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True),
                                                      y_types[0], y_types[1],
                                                      path=adq.PATH_SPLIT)
    ex.set_split(0, launches)
    ref_ex, ref = adq.plan_add_rms_norm_dynamic_quant_v2(
        x1, x2, g, b, s1, s2, 1e-6, (True, True), y_types[0], y_types[1], path=adq.PATH_SPLIT)
    ref_ex.set_split(0, launches)
    assert ex.describe() == ref_ex.describe() and f"launches={launches}" in ex.describe()
    ws = torch.empty(ex.workspace_size, dtype=torch.uint8, device="cuda")
    ref_ws = torch.empty(ex.workspace_size, dtype=torch.uint8, device="cuda")
    graph = capture(lambda: ex.run(ws))
    previous = None
    for rep in range(REPLAYS):
        n1, n2 = synth.inputs(w, seed=700 + rep)
        x1.copy_(dev(n1, dtype))
        x2.copy_(dev(n2, dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(outs[k]) for k in ("x_out", "y1", "y2", "scale1", "scale2")]
        ref_ex.run(ref_ws)
        torch.cuda.synchronize()
        want = [bits(ref[k]) for k in ("x_out", "y1", "y2", "scale1", "scale2")]
        for a_, b_ in zip(got, want):
            assert np.array_equal(a_, b_), f"replay {rep} differs from the eager call"
        assert previous is None or not np.array_equal(got[1], previous), "replay saw stale inputs"
        previous = got[1]
    ex.close()
    ref_ex.close()


def test_rms_norm_dq_replays_match_eager():
    w = synth.Workload("graph", "rmsnorm", 64, 1024, "fp16", 78, None, False, 1)
    g, _, s1, _ = synth.params(w)
    g, s1 = dev(g, "fp16"), dev(s1, "fp16")
    x = dev(synth.inputs(w)[0], "fp16")
    ex, outs = adq.plan_rms_norm_dynamic_quant(x, g, None, s1, 1e-6, "int4")
    graph = capture(lambda: ex.run(None))
    for rep in range(REPLAYS):
        x.copy_(dev(synth.inputs(w, seed=600 + rep)[0], "fp16"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (bits(outs["y"]), bits(outs["scale"]))
        y, sc = adq.rms_norm_dynamic_quant(x, g, None, s1, 1e-6, "int4")
        torch.cuda.synchronize()
        assert np.array_equal(got[0], bits(y)) and np.array_equal(got[1], bits(sc)), rep
    ex.close()


def test_gemm_replays_match_eager():
    rng = np.random.default_rng(79)
    m, n, k = 300, 520, 256
    a = torch.from_numpy(rng.integers(-127, 128, (m, k)).astype(np.int8)).cuda()
    w = torch.from_numpy(rng.integers(-127, 128, (n, k)).astype(np.int8)).cuda()
    sa = torch.from_numpy(rng.uniform(0.01, 0.08, m).astype(np.float32)).cuda()
    sw = torch.from_numpy(rng.uniform(1e-4, 1e-3, n).astype(np.float32)).cuda()
    bias = torch.from_numpy(rng.normal(0, 0.1, n).astype(np.float32)).cuda()
    ex, out = adq.plan_w8a8_gemm(a, sa, w, sw, bias, out_dtype=torch.bfloat16)
    graph = capture(lambda: ex.run(None))
    for rep in range(REPLAYS):
        a.copy_(torch.from_numpy(rng.integers(-127, 128, (m, k)).astype(np.int8)).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(out)
        ref = adq.w8a8_gemm(a, sa, w, sw, bias, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(got, bits(ref)), rep
    ex.close()


@pytest.mark.parametrize("rows,rank", [(300, 16), (700, 16), (700, 64)],
                         ids=["grouping_in_shrink", "grouping_launch", "mfma_expand"])
def test_lora_replays_match_eager(rows, rank):
    """Both tiled launch sequences, and the matrix-core expand (bf16, rank
    64); the workspace holds the previous replay's table and partial sums,
    which every launch rewrites before reading."""
    h1, h2, h3, wn, layers, layer, off, dt = 256, 192, 320, 5, 2, 1, 64, "bf16"
    s = 80 + rows
    td = torch.bfloat16
    t = lambda bits_: torch.from_numpy(np.ascontiguousarray(bits_).view(np.int16)).view(td).cuda()
    y = t(small_ints(s, 13, (rows, h3), -8, 8, dt))
    x = t(small_ints(s, 12, (rows, h1), -2, 2, dt))
    wa = t(small_ints(s, 14, (wn, layers, h1, rank), -2, 2, dt))
    wb = t(small_ints(s, 15, (wn, layers, rank, h2), -2, 2, dt))
    idx = torch.from_numpy(synth.int32s(s, 16, -1, wn, rows)).cuda()
    out = torch.empty_like(y)
    ex, out = adq.plan_add_lora(y, x, wb, idx, wa, layer, 0.5, off, out=out)
    assert "lora-tiled" in ex.describe()
    ws = torch.empty(ex.workspace_size, dtype=torch.uint8, device="cuda")
    graph = capture(lambda: ex.run(ws))
    for rep in range(REPLAYS):
        x.copy_(t(small_ints(s + 1 + rep, 12, (rows, h1), -2, 2, dt)))
        idx.copy_(torch.from_numpy(synth.int32s(s + 1 + rep, 16, -1, wn, rows)).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(out)
        ref = adq.add_lora(y, x, wb, idx, wa, layer, 0.5, off)
        torch.cuda.synchronize()
        assert np.array_equal(got, bits(ref)), rep
    ex.close()
