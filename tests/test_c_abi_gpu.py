"""The C-ABI from plain C: tests/c_driver/adq_c_driver.c (built by
__graft_entry__.build()) calls the two-phase AddRmsNormDynamicQuantV2
functions of include/adq.h with hipMalloc'd memory on its own HIP stream,
in its own process, and checks phase 1's error report for a missing input;
in its second mode it sets the split-row path's one-launch form with
adq_executor_set_split and runs the executor through both run entry points
(with a workspace, and the one that allocates nothing), requiring the same
bytes; its outputs are checked here against the oracle under the parity
rules."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from helpers import check_codes, check_scales, unpack_int4

pytestmark = pytest.mark.gpu
DRIVER = os.path.join(os.path.dirname(__file__), "c_driver", "adq_c_driver")


@pytest.mark.parametrize("m,n,dtype,mode", [(37, 4096, "bf16", 0), (300, 24584, "fp16", 0),
                                            (32, 16384, "bf16", 1), (5, 40008, "fp16", 1)])
def test_c_caller_matches_oracle(tmp_path, m, n, dtype, mode):
    assert os.path.exists(DRIVER), "run __graft_entry__.build() first"
    w = synth.Workload("c_abi", "v2", m, n, dtype, 31, (True, True), True, 2, ("int8", "int4"))
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    for name, arr in (("x1", x1), ("x2", x2), ("gamma", g), ("beta", b), ("s1", s1), ("s2", s2)):
        np.ascontiguousarray(arr).astype(np.uint16).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "shape.txt").write_text(f"{m} {n} {2 if dtype == 'bf16' else 1} {mode}\n")
    print(f"\n[case] C driver {m}x{n} {dtype} mode {mode}", flush=True)
    r = subprocess.run([DRIVER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("ok"), r.stdout
    if mode == 1:
        assert "path=split" in r.stdout and "launches=1" in r.stdout, r.stdout
    ora = oracle.add_rms_norm_dq_v2(x1, x2, g, b, s1, s2, 1e-6, (True, True), "int8", "int4",
                                    dtype)
    xo = np.fromfile(tmp_path / "xout.bin", dtype=np.uint16).reshape(m, n)
    assert np.array_equal(xo, ora["x_out"]), "xOut differs"
    check_scales(np.fromfile(tmp_path / "scale1.bin", dtype=np.float32), ora["scale1"])
    check_scales(np.fromfile(tmp_path / "scale2.bin", dtype=np.float32), ora["scale2"])
    y1 = np.fromfile(tmp_path / "y1.bin", dtype=np.int8).reshape(m, n)
    y2 = np.fromfile(tmp_path / "y2.bin", dtype=np.uint8).reshape(m, n // 2)
    check_codes(y1, ora["code1"], ora["pre1"])
    check_codes(unpack_int4(y2), ora["code2"], ora["pre2"])
