"""bench.py on the CPU: algorithmic-byte accounting of every workload, and
the single-GPU contract of its command line."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# bytes per launch: inputs read once + outputs written once + parameter vectors once,
# worked out by hand for each workload
EXPECTED = {
    # 64 rows * (2*1024 read + 1024 + 4) + gamma 2*1024
    "rmsnorm_dq": ([True, False], 64 * (2 * 1024 + 1024 + 4) + 2 * 1024),
    # 4096 * (2*2*4096 + 2*4096 + 4096 + 4) + (gamma, beta, s1) 3*2*4096
    "v2_square": ([True, False], 4096 * (4 * 4096 + 2 * 4096 + 4096 + 4) + 3 * 2 * 4096),
    # 32 * (4*16384 + 2*16384 + 2*(16384 + 4)) + 4*2*16384
    "v2_decode": ([True, True], 32 * (4 * 16384 + 2 * 16384 + 2 * (16384 + 4)) + 4 * 2 * 16384),
    "v2_outlier": ([True, True], 16384 * (4 * 8192 + 2 * 8192 + 2 * (8192 + 4)) + 4 * 2 * 8192),
    # INT4: 5120/2 bytes of codes per row
    "v2_int4": ([True, False], 65536 * (4 * 5120 + 2 * 5120 + 2560 + 4) + 3 * 2 * 5120),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes(name):
    active, want = EXPECTED[name]
    assert bench.alg_bytes(synth.WORKLOADS[name], active) == want


def test_headline_bytes_value():
    assert bench.alg_bytes(synth.WORKLOADS["v2_outlier"], [True, True]) == 1_073_938_432


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_matches_its_hash_or_is_ignored():
    t = bench.measured_traffic("v2_outlier")
    assert t is None or t > bench.alg_bytes(synth.WORKLOADS["v2_outlier"], [True, True]) * 0.99
    assert bench.measured_traffic("no_such_workload") is None


def test_threaded_wall_covers_every_item_once():
    seen = []
    import threading
    lock = threading.Lock()

    def part(lo, hi):
        with lock:
            seen.extend(range(lo, hi))

    for n, t in ((10, 3), (7, 16), (1, 4), (64, 8)):
        seen.clear()
        assert bench.threaded_wall(part, n, t) >= 0.0
        assert sorted(seen) == list(range(n))


def test_host_threads_is_bounded():
    assert 1 <= bench.host_threads() <= 16


def test_lora_algorithmic_bytes_by_hand():
    # lora_prefill: every row has an adapter (indices drawn from [0, 8)):
    # x 4096*4096*2 + y slice read and written 2*4096*4096*2 + indices 4*4096
    # + 8 adapters' layer weights (4096*16 + 16*4096) * 2
    wl = synth.LORA_WORKLOADS["lora_prefill"]
    idx = synth.lora_inputs(wl)[4]
    assert ((idx >= 0) & (idx < wl.w)).all() and len(set(idx.tolist())) == 8
    want = 4096 * 4096 * 2 + 2 * 4096 * 4096 * 2 + 4 * 4096 + 8 * (4096 * 16 + 16 * 4096) * 2
    assert bench.lora_alg_bytes(wl, idx) == want == 102_776_832


class _FakeCuda:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


class _FakeTorch:
    def __init__(self):
        self.cuda = _FakeCuda()


def test_settle_runs_the_warmup_count_and_the_time_floor():
    """The untimed phase makes at least `warmup` launches, goes on until the
    time floor has passed, keeps the host in step with the device, and ends
    with a synchronization (so the timed launches start on an idle queue)."""
    import time
    calls = []
    torch = _FakeTorch()
    n = bench.settle(torch, lambda i: calls.append(i), 40, 0.0)
    assert n == 40 and calls == list(range(40))
    assert torch.cuda.syncs >= 40 // 16 + 1

    calls.clear()
    torch = _FakeTorch()
    t0 = time.perf_counter()
    n = bench.settle(torch, lambda i: (calls.append(i), time.sleep(0.001)), 3, 30.0)
    assert (time.perf_counter() - t0) * 1e3 >= 30.0
    assert n == len(calls) and n > 3
    assert torch.cuda.syncs >= n // 16
