"""Benchmark of the fused AddRmsNorm + per-row dynamic quantization kernel.

One step = one launch of the whole operator (load + add + xOut, RmsNorm,
smooth scaling, row maxima, scales, quantize + pack + store) over one batch
of synthetic inputs already resident in HBM.  The default workload is
AddRmsNormDynamicQuantV2 on bf16 [16384, 8192] with 1% outlier columns,
two smooth scales and two INT8 outputs (plus scales and xOut).

Prints ONE JSON line with the achieved HBM bandwidth (algorithmic bytes /
average launch time, HIP events on the launch stream), its fraction of the
MI355X HBM3E peak, and the CPU oracle timed on a bounded sample of the same
workload on the host cores.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload v2_outlier]

``--workload w8a8_gemm`` instead times the INT8 GEMM that consumes the
quantized rows (16384 x 8192 codes with per-row scales through an
8192 -> 8192 projection with per-column weight scales, bf16 out) against
the MI355X dense INT8 MFMA peak (``--gemm-rows M`` runs it with M rows of
activations; few rows are bound by reading the weights and are reported
against HBM bandwidth).  ``--workload lora_prefill`` (or
lora_decode) times AddLora accumulating into y in place, against HBM
bandwidth; ``--lora-rank R`` runs it at another rank.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0  # MI355X dense INT8 MFMA, 5.0 POP/s
SETTLE_MS = 50.0  # least time of untimed launches before a timed run


def alg_bytes(w, active, rows=None):
    """Bytes the operator must move: inputs read once, outputs written once,
    parameter vectors read once.  `active`: which quantized outputs exist."""
    rows = w.rows if rows is None else rows
    n, b = w.cols, 2
    n_in = 2 if w.op == "v2" else 1
    per_row = n_in * b * n + (b * n if w.op == "v2" else 0)
    for k, act in enumerate(active):
        if act:
            bits = 4 if w.y_types[k] == "int4" else 8
            per_row += n * bits // 8 + 4
    params = (1 + int(w.has_beta) + w.n_smooth) * b * n
    return rows * per_row + params


# Sources that determine each path's kernels and launch plans (a traffic
# record is valid only for the sources it was measured on).
_COMMON_SOURCES = ["adq_device.h", "adq_internal.h", "adq_api.cpp"]
_PATH_SOURCES = {
    "operator": ["adq_row_impl.h", "adq_row_bf16.hip", "adq_row_f16.hip", "adq_split.hip",
                 "adq_generic.hip"],
    "gemm": ["adq_gemm.hip"],
    "lora": ["adq_lora.hip"],
}


def path_of(workload: str) -> str:
    """Kernel family of a workload, also of the names derived from one
    (w8a8_gemm_m32: another row count; lora_prefill_rank64: another rank)."""
    import synth
    if workload.startswith(tuple(synth.GEMM_WORKLOADS)):
        return "gemm"
    return "lora" if workload.startswith(tuple(synth.LORA_WORKLOADS)) else "operator"


def kernel_source_hash(workload: str = "v2_outlier") -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_dynamic_quantization_amd", "csrc")
    for name in sorted(_COMMON_SOURCES + _PATH_SOURCES[path_of(workload)]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(workload):
        return None
    return t.get("hbm_bytes_per_launch")


def host_threads() -> int:
    """Host cores this process may use (at most 16: one GPU's share of the
    host), for the multi-threaded oracle leg."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def threaded_wall(fn, n_items: int, threads: int) -> float:
    """Wall time of fn(lo, hi) over [0, n_items) cut into `threads`
    contiguous parts run at once (the oracle's C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    parts = [(n_items * i // threads, n_items * (i + 1) // threads) for i in range(threads)]
    parts = [p for p in parts if p[1] > p[0]]
    with ThreadPoolExecutor(len(parts)) as pool:
        t0 = time.perf_counter()
        list(pool.map(lambda p: fn(*p), parts))
        return time.perf_counter() - t0


def timed_copy_us(torch, nbytes: int, steps: int = 20) -> float:
    """Average time of a plain device copy of `nbytes` bytes (torch's copy
    kernel), HIP events around back-to-back copies, rotating through enough
    buffer pairs that every copy streams from HBM."""
    sets = max(1, math.ceil(512e6 / (2 * nbytes)))
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")) for _ in range(sets)]
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: bufs[i % sets][1].copy_(bufs[i % sets][0]), 3, SETTLE_MS)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        bufs[i % sets][1].copy_(bufs[i % sets][0])
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / steps * 1e3
    del bufs
    torch.cuda.empty_cache()
    return us


def device_context(torch, step_bytes: int) -> dict:
    """The device's own figures, as context for the bandwidth numbers: the
    memory clock and bus width it reports, a plain 1 GiB device copy, and a
    plain copy moving the same number of bytes as one step (half read, half
    written), both timed with HIP events as read + write bytes / time."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    ctx = {"device": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        # hipDeviceAttributeMemoryBusWidth = 59, hipDeviceAttributeMemoryClockRate = 60
        # (kHz) in hip_runtime_api.h of ROCm 7
        val = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 59, torch.cuda.current_device()) == 0:
            ctx["memory_bus_bits"] = val.value
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 60, torch.cuda.current_device()) == 0:
            ctx["memory_clock_mhz"] = val.value / 1000
    except OSError:
        pass
    us = timed_copy_us(torch, 1 << 29)
    ctx["copy_1gib_gbs"] = round(2 * (1 << 29) / us / 1e3, 1)
    if step_bytes > 0:
        half = step_bytes // 2
        us = timed_copy_us(torch, half)
        ctx["copy_same_bytes"] = {"bytes": 2 * half, "us": round(us, 1),
                                  "gbs": round(2 * half / us / 1e3, 1)}
    return ctx


def make_cases(w, torch, adq, synth, dev, path, n_sets, split=(0, 0)):
    """n_sets independent input/output sets of a workload (inputs uploaded
    once and copied on the device), each with its executor and workspace;
    returns (cases, host inputs, active outputs)."""
    x1, x2 = synth.inputs(w)
    g, b, s1, s2 = synth.params(w)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
    d = lambda a: None if a is None else torch.from_numpy(a.view("int16")).view(td).to(dev)
    base1, base2 = d(x1), d(x2)
    params = [d(p) for p in (g, b, s1, s2)]
    cases = []
    for i in range(n_sets):
        t1 = base1 if i == 0 else base1.clone()
        t2 = None if base2 is None else (base2 if i == 0 else base2.clone())
        if w.op == "v2":
            ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
                t1, t2, *params, w.eps, w.mask, w.y_types[0], w.y_types[1], path=path)
        else:
            ex, outs = adq.plan_rms_norm_dynamic_quant(t1, params[0], params[1], params[2],
                                                       w.eps, w.y_types[0], path=path)
        if path == adq.PATH_SPLIT and any(split):
            ex.set_split(split[0], split[1])
        ws = (torch.empty(ex.workspace_size, dtype=torch.uint8, device=dev)
              if ex.workspace_size else None)
        cases.append((ex, ws, outs))
    if w.op == "v2":
        active = [cases[0][2]["y1"] is not None, cases[0][2]["y2"] is not None]
    else:
        active = [True, False]
    return cases, (x1, x2, g, b, s1, s2), active


def active_outputs(w):
    """Which quantized outputs a workload produces (the V2 page's cases)."""
    if w.op != "v2":
        return [True, False]
    if w.mask is not None:
        return [bool(w.mask[0]), bool(w.mask[1])]
    return [True, w.n_smooth >= 2]


def settle(torch, launch, warmup, settle_ms):
    """`warmup` launches, continued until at least `settle_ms` of back-to-back
    launches have run: after an idle spell the GPU needs about 20 ms of
    sustained load before its launch time settles (bf16 16384 x 8192, windows
    of 10 launches after 0.5 s idle: 172 us, rising to 195 us by the 30th
    launch, back to 165 us from about the 100th on).  Returns the number of
    launches made."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        launch(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()  # keeps the host clock on the GPU's work
    torch.cuda.synchronize()
    return i


def time_operator(w, torch, adq, synth, path, steps, warmup, rotate=True, keep=False,
                  split=(0, 0), settle_ms=SETTLE_MS):
    """Average launch time of one operator workload: `steps` back-to-back
    launches between two HIP events on the launch stream, after `warmup`
    launches that go on for at least `settle_ms`, rotating through enough
    input/output sets that every launch streams from HBM rather than the
    256 MB last-level cache."""
    dev = torch.device("cuda:0")
    footprint = alg_bytes(w, active_outputs(w))
    n_sets = max(1, math.ceil(512e6 / footprint)) if rotate else 1
    cases, host_inputs, active = make_cases(w, torch, adq, synth, dev, path, n_sets, split)
    stream = torch.cuda.current_stream()

    def launch(i):
        ex, ws, _ = cases[i % n_sets]
        ex.run(ws, stream)

    warm = settle(torch, launch, warmup, settle_ms)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ex, ws, _ = cases[i % n_sets]
        ex.run(ws, stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    plan = cases[0][0].describe()
    res = {"ms": ms, "wall": wall, "bytes": footprint, "sets": n_sets, "plan": plan,
           "active": active, "host_inputs": host_inputs if keep else None, "warm": warm}
    for ex, _, _ in cases:
        ex.close()
    del cases
    torch.cuda.empty_cache()
    return res


def config_entry(w, r, steps):
    """Per-workload figures for the bench line's `configs` object."""
    us = r["ms"] * 1e3
    gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
    return {
        "op": "AddRmsNormDynamicQuantV2" if w.op == "v2" else "RmsNormDynamicQuant",
        "rows": w.rows, "cols": w.cols, "storage": w.dtype,
        "outputs": [t for t, a in zip(w.y_types, r["active"]) if a],
        "algorithmic_bytes": r["bytes"], "launches_timed": steps, "untimed_launches": r["warm"],
        "rotating_sets": r["sets"],
        "us_per_launch": round(us, 2), "gbs": round(gbs, 1),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "rows_per_s": round(w.rows / (r["ms"] * 1e-3)),
        "kernel_path": r["plan"].split()[0].split("=")[1],
        "plan": " ".join(x for x in r["plan"].split()
                         if x.split("=")[0] in ("vpt", "block", "grid", "splits", "launches")),
        "traffic": measured_traffic(w.name),
    }


def cpu_baseline(w, active, host_inputs, budget_s: float):
    """The oracle (plain C, one thread) on the first rows of the same inputs,
    as many rows as fit the time budget after a short pilot."""
    import oracle
    x1, x2, g, b, s1, s2 = host_inputs

    def run(rows):
        t0 = time.perf_counter()
        if w.op == "v2":
            oracle.add_rms_norm_dq_v2(x1[:rows], x2[:rows], g, b, s1, s2, w.eps, w.mask,
                                      w.y_types[0], w.y_types[1], w.dtype, want_pre=False)
        else:
            oracle.rms_norm_dq(x1[:rows], g, b, s1, w.eps, w.y_types[0], w.dtype,
                               want_pre=False)
        return time.perf_counter() - t0

    def run_part(lo, hi):
        if w.op == "v2":
            oracle.add_rms_norm_dq_v2(x1[lo:hi], x2[lo:hi], g, b, s1, s2, w.eps, w.mask,
                                      w.y_types[0], w.y_types[1], w.dtype, want_pre=False)
        else:
            oracle.rms_norm_dq(x1[lo:hi], g, b, s1, w.eps, w.y_types[0], w.dtype,
                               want_pre=False)

    pilot = min(w.rows, 16)
    t = run(pilot)
    rows = int(max(pilot, min(w.rows, budget_s / max(t / pilot, 1e-9))))
    t = run(rows)
    gbs = alg_bytes(w, active, rows) / t / 1e9
    single = {"value": round(gbs, 4), "cores": 1,
              "sample": f"first {rows} of {w.rows} rows, {t:.2f} s ({rows / t:.0f} rows/s)"}
    # the same oracle, rows split over the host's cores
    threads = host_threads()
    rows_mt = min(w.rows, rows * threads)
    t_mt = threaded_wall(run_part, rows_mt, threads)
    gbs_mt = alg_bytes(w, active, rows_mt) / t_mt / 1e9
    return {"value": round(gbs_mt, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows_mt} of {w.rows} rows of the same seeded inputs split over "
                      f"{threads} threads, {t_mt:.2f} s wall, plain-C fp64 oracle "
                      f"({rows_mt / t_mt:.0f} rows/s)",
            "single_thread": single}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed launches before the timed ones; they go on for at least "
                         f"{SETTLE_MS:.0f} ms however many that takes")
    ap.add_argument("--workload", default="v2_outlier")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--path", choices=["auto", "row", "split", "generic"], default="auto",
                    help="kernel path (default: the library's own choice)")
    ap.add_argument("--splits", type=int, default=0, metavar="S",
                    help="with --path split: S chunks per row (0 = the planner's choice)")
    ap.add_argument("--launches", type=int, default=0, choices=[0, 1, 2, 3],
                    help="with --path split: the one-, two- or three-launch form (0 = the "
                         "planner's choice)")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the chosen workload (by default every operator workload "
                         "is also timed and reported under `configs`)")
    ap.add_argument("--no-rotate", action="store_true",
                    help="reuse one input/output set (cache-warm) instead of rotating sets "
                         "that do not fit the last-level cache")
    ap.add_argument("--gemm-rows", type=int, default=0, metavar="M",
                    help="with --workload w8a8_gemm: M rows of activations instead of 16384 "
                         "(few rows are bound by reading the weights; the bench line then "
                         "reports HBM GB/s)")
    ap.add_argument("--lora-rank", type=int, default=0, metavar="R",
                    help="AddLora workloads: use rank R (8, 16, 32, 64, 128 take the tiled "
                         "kernels) instead of the workload's own")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead: time a plain device-to-device copy of MIB MiB (reference "
                         "for achievable bandwidth and for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the operator is row-local and the library runs on a "
              f"single MI355X, so --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy, args.steps, args.warmup)
        return
    import int4_dynamic_quantization_amd as adq
    import synth

    if args.workload in synth.GEMM_WORKLOADS:
        bench_gemm(args, torch, adq, synth)
        return
    if args.workload in synth.LORA_WORKLOADS:
        bench_lora(args, torch, adq, synth)
        return
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    path = {"auto": adq.PATH_AUTO, "row": adq.PATH_ROW, "split": adq.PATH_SPLIT,
            "generic": adq.PATH_GENERIC}[args.path]
    footprint = alg_bytes(w, active_outputs(w))
    print(f"[bench] workload {w.name} {w.rows}x{w.cols} {w.dtype}: {footprint / 1e6:.1f} MB "
          f"per launch", file=sys.stderr, flush=True)
    head = time_operator(w, torch, adq, synth, path, args.steps, args.warmup,
                         rotate=not args.no_rotate, keep=args.cpu_budget > 0,
                         split=(args.splits, args.launches))
    ms = head["ms"]
    gbs = footprint / (ms * 1e-3) / 1e9
    print(f"[bench] plan: {head['plan']}", file=sys.stderr, flush=True)
    print(f"[bench] {args.steps} launches: avg {ms * 1e3:.1f} us per launch, "
          f"wall {head['wall'] * 1e3:.1f} ms", file=sys.stderr, flush=True)
    n_sets = head["sets"]
    active = head["active"]

    traffic = measured_traffic(w.name)
    result = {
        "metric": "achieved HBM GB/s (% of peak), AddRmsNorm+DynQuant bf16 16384x8192",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "op": "AddRmsNormDynamicQuantV2" if w.op == "v2" else "RmsNormDynamicQuant",
            "rows": w.rows, "cols": w.cols, "storage": w.dtype,
            "outputs": [t for t, a in zip(w.y_types, active) if a],
            "outlier_columns": w.n_outlier, "smooth_scales": w.n_smooth,
            "algorithmic_bytes_per_step": footprint,
            "rows_per_s": round(w.rows / (ms * 1e-3)),
            "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "parallelism": "single GPU",
            "kernel_path": head["plan"].split()[0].split("=")[1],
            "plan": " ".join(x for x in head["plan"].split()
                             if x.split("=")[0] in ("vpt", "block", "grid", "splits", "launches",
                                                    "store")),
            "untimed_launches": head["warm"],
            "settle_ms": SETTLE_MS,
            "cache": "warm (one set)" if n_sets == 1 and args.no_rotate else
                     f"cold ({n_sets} rotating sets)" if n_sets > 1 else "cold (footprint > LLC)",
        },
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not args.no_configs:
        # every workload of the operator, measured the same way (the headline
        # among them, in a run of its own)
        configs = {}
        for name, wc in synth.WORKLOADS.items():
            steps = args.steps if alg_bytes(wc, active_outputs(wc)) >= 100e6 else max(args.steps, 1000)
            r = time_operator(wc, torch, adq, synth, adq.PATH_AUTO, steps, args.warmup)
            configs[name] = config_entry(wc, r, steps)
            print(f"[bench] config {name}: {configs[name]['us_per_launch']} us, "
                  f"{configs[name]['gbs']} GB/s ({configs[name]['kernel_path']})",
                  file=sys.stderr, flush=True)
        result["configs"] = configs
    result["context"] = device_context(torch, footprint)
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(w, active, head["host_inputs"], args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def gemm_cpu_baseline(a, sa, w, sw, b, k: int, budget_s: float, step_bytes: int = 0):
    """The oracle (plain C, one thread, exact int64 sums) on a sample of the
    outputs, as many as fit the time budget after a short pilot.  In TOPS;
    with `step_bytes`, in GB/s instead: the step's bytes times the share of
    its outputs computed per second."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)

    def run(count):
        rows = rng.integers(0, a.shape[0], count)
        cols = rng.integers(0, w.shape[0], count)
        t0 = time.perf_counter()
        oracle.w8a8_gemm_at(a, sa, w, sw, b, rows, cols)
        return time.perf_counter() - t0

    pilot = 256
    t = run(pilot)
    count = int(max(pilot, budget_s / max(t / pilot, 1e-9)))
    t = run(count)
    outputs = a.shape[0] * w.shape[0]
    rate = lambda c, secs: (step_bytes * c / outputs / secs / 1e9 if step_bytes
                            else 2.0 * k * c / secs / 1e12)
    single = {"value": round(rate(count, t), 6), "cores": 1,
              "sample": f"{count} randomly placed outputs, {t:.2f} s"}
    # the same oracle, the sampled outputs split over the host's cores
    threads = host_threads()
    count_mt = count * threads
    rows = rng.integers(0, a.shape[0], count_mt)
    cols = rng.integers(0, w.shape[0], count_mt)
    t_mt = threaded_wall(lambda lo, hi: oracle.w8a8_gemm_at(a, sa, w, sw, b, rows[lo:hi],
                                                            cols[lo:hi]), count_mt, threads)
    return {"value": round(rate(count_mt, t_mt), 6), "unit": "GB/s" if step_bytes else "TOPS",
            "cores": threads, "kind": "oracle",
            "sample": f"{count_mt} randomly placed outputs of the same seeded inputs "
                      f"(2*k ops each) split over {threads} threads, {t_mt:.2f} s wall, "
                      f"plain-C int64 oracle" +
                      (f"; as GB/s: {step_bytes} bytes per step times the share of the "
                       f"step's {outputs} outputs done per second" if step_bytes else ""),
            "single_thread": single}


def bench_gemm(args, torch, adq, synth) -> None:
    """One step = one launch of the INT8 GEMM with its dequantizing epilogue."""
    w8 = synth.GEMM_WORKLOADS[args.workload]
    if args.gemm_rows:
        w8 = dataclasses.replace(w8, name=f"{w8.name}_m{args.gemm_rows}", m=args.gemm_rows)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a, sa, wq, sw, b = synth.gemm_inputs(w8)
    t = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    out_dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "f32": torch.float32}[w8.out_dtype]
    ex, out = adq.plan_w8a8_gemm(t(a), t(sa), t(wq), t(sw), t(b), out_dtype=out_dt)
    print(f"[bench] workload {w8.name} m={w8.m} n={w8.n} k={w8.k} out {w8.out_dtype}; "
          f"plan: {ex.describe()}", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: ex.run(None, stream), args.warmup, SETTLE_MS)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        ex.run(None, stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    ops = 2.0 * w8.m * w8.n * w8.k
    tops = ops / (ms * 1e-3) / 1e12
    # bytes the product must move: both operands, the scales (and bias), the output
    out_bytes = {"bf16": 2, "fp16": 2, "f32": 4}[w8.out_dtype]
    nbytes = (w8.m * w8.k + w8.n * w8.k + 4 * w8.m + 4 * w8.n * (2 if w8.has_bias else 1) +
              out_bytes * w8.m * w8.n)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the roofline of whichever resource bounds the shape: matrix cores for
    # many rows, reading the weights for few
    mfma_bound = ops / (INT8_PEAK_TOPS * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9)
    print(f"[bench] {args.steps} launches: avg {ms * 1e3:.1f} us per launch, "
          f"wall {wall * 1e3:.1f} ms", file=sys.stderr, flush=True)
    result = {
        "metric": (f"achieved INT8 TOPS (% of dense MFMA peak), W8A8 GEMM "
                   f"{w8.m}x{w8.n}x{w8.k}" if mfma_bound else
                   f"achieved HBM GB/s (% of peak), W8A8 GEMM {w8.m}x{w8.n}x{w8.k}"),
        "value": round(tops, 1) if mfma_bound else round(gbs, 1),
        "unit": "TOPS" if mfma_bound else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": w8.name, "op": "W8A8 GEMM (per-row x per-column scales)",
            "m": w8.m, "n": w8.n, "k": w8.k, "out": w8.out_dtype, "bias": w8.has_bias,
            "algorithmic_ops_per_step": ops, "algorithmic_bytes_per_step": nbytes,
            "tops": round(tops, 1), "gbs": round(gbs, 1),
            "pct_of_peak": round(100 * tops / INT8_PEAK_TOPS, 2) if mfma_bound else
                           round(100 * gbs / HBM_PEAK_GBS, 2),
            "parallelism": "single GPU",
            "plan": ex.describe(),
        },
        "roofline": ({"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS,
                      "unit": "TOPS", "frac": round(tops / INT8_PEAK_TOPS, 4),
                      "traffic": measured_traffic(w8.name)} if mfma_bound else
                     {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic(w8.name)}),
    }
    ex.close()
    result["context"] = device_context(torch, 0)
    result["cpu_baseline"] = (gemm_cpu_baseline(a, sa, wq, sw, b, w8.k, args.cpu_budget,
                                                0 if mfma_bound else nbytes)
                              if args.cpu_budget > 0 else None)
    print(json.dumps(result), flush=True)


def lora_alg_bytes(wl, idx, in_place=True) -> int:
    """Bytes AddLora must move: x read, y's slice read and written (the whole
    of y read and out written when out is not y), the index vector, and the
    layer's weights of each adapter that some row uses."""
    import numpy as np
    b = 2
    used = len(set(int(g) for g in np.unique(idx) if 0 <= g < wl.w))
    per_adapter = (wl.h1 * wl.rank if wl.has_a else 0) + wl.rank * wl.h2
    rows_with = int(((idx >= 0) & (idx < wl.w)).sum())
    y_bytes = 2 * rows_with * wl.h2 * b if in_place else 2 * wl.rows * wl.h3 * b
    return (rows_with * wl.h1 * b + y_bytes + 4 * wl.rows + used * per_adapter * b)


def lora_cpu_baseline(wl, host, alg_rows_bytes, budget_s: float):
    """The oracle (plain C, one thread) on the first rows of the same inputs."""
    import oracle
    y, x, wa, wb, idx = host

    def run(rows):
        t0 = time.perf_counter()
        oracle.add_lora(y[:rows], x[:rows], wb, idx[:rows], wa, wl.layer, wl.scale, wl.y_offset,
                        wl.dtype, want_pre=False)
        return time.perf_counter() - t0

    pilot = min(wl.rows, 4)
    t = run(pilot)
    rows = int(max(pilot, min(wl.rows, budget_s / max(t / pilot, 1e-9))))
    t = run(rows)
    gbs = alg_rows_bytes * rows / wl.rows / t / 1e9
    single = {"value": round(gbs, 5), "cores": 1,
              "sample": f"first {rows} of {wl.rows} rows, {t:.2f} s ({rows / t:.1f} rows/s)"}
    # the same oracle, rows split over the host's cores
    threads = host_threads()
    rows_mt = min(wl.rows, rows * threads)
    t_mt = threaded_wall(lambda lo, hi: oracle.add_lora(
        y[lo:hi], x[lo:hi], wb, idx[lo:hi], wa, wl.layer, wl.scale, wl.y_offset, wl.dtype,
        want_pre=False), rows_mt, threads)
    gbs_mt = alg_rows_bytes * rows_mt / wl.rows / t_mt / 1e9
    return {"value": round(gbs_mt, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows_mt} of {wl.rows} rows of the same seeded inputs split over "
                      f"{threads} threads, {t_mt:.2f} s wall, plain-C fp64 oracle "
                      f"({rows_mt / t_mt:.1f} rows/s)",
            "single_thread": single}


def bench_lora(args, torch, adq, synth) -> None:
    """One step = one AddLora launch accumulating into y in place."""
    wl = synth.LORA_WORKLOADS[args.workload]
    if args.lora_rank and args.lora_rank != wl.rank:
        wl = dataclasses.replace(wl, name=f"{wl.name}_rank{args.lora_rank}", rank=args.lora_rank)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host = synth.lora_inputs(wl)
    y, x, wa, wb, idx = host
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    d = lambda a: None if a is None else torch.from_numpy(a.view("int16")).view(td).to(dev)
    alg = lora_alg_bytes(wl, idx)
    n_sets = 1 if args.no_rotate else max(1, math.ceil(512e6 / alg))
    tw = (d(wb), d(wa), torch.from_numpy(idx).to(dev))
    cases = []
    for _ in range(n_sets):
        ty, tx = d(y), d(x)
        ex, _ = adq.plan_add_lora(ty, tx, tw[0], tw[2], tw[1], wl.layer, wl.scale, wl.y_offset,
                                  out=ty, path=adq.PATH_GENERIC if args.path == "generic"
                                  else adq.PATH_AUTO)
        ws = (torch.empty(ex.workspace_size, dtype=torch.uint8, device=dev)
              if ex.workspace_size else None)
        cases.append((ex, ws, ty, tx))
    print(f"[bench] workload {wl.name}: {alg / 1e6:.1f} MB per launch, {n_sets} rotating set(s); "
          f"plan: {cases[0][0].describe()}", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: cases[i % n_sets][0].run(cases[i % n_sets][1], stream), args.warmup,
           SETTLE_MS)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        cases[i % n_sets][0].run(cases[i % n_sets][1], stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    gbs = alg / (ms * 1e-3) / 1e9
    print(f"[bench] {args.steps} launches: avg {ms * 1e3:.1f} us per launch, "
          f"wall {wall * 1e3:.1f} ms", file=sys.stderr, flush=True)
    result = {
        "metric": f"achieved HBM GB/s (% of peak), AddLora {wl.dtype} {wl.rows} rows "
                  f"{wl.h1}->{wl.rank}->{wl.h2}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "op": "AddLora (in place)", "rows": wl.rows, "h1": wl.h1,
            "rank": wl.rank, "h2": wl.h2, "h3": wl.h3, "adapters": wl.w, "layers": wl.l,
            "storage": wl.dtype, "algorithmic_bytes_per_step": alg,
            "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "parallelism": "single GPU", "plan": cases[0][0].describe(),
            "cache": "warm (one set)" if n_sets == 1 else f"cold ({n_sets} rotating sets)",
        },
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name)},
    }
    for ex, _, _, _ in cases:
        ex.close()
    result["context"] = device_context(torch, alg)
    result["cpu_baseline"] = (lora_cpu_baseline(wl, host, alg, args.cpu_budget)
                              if args.cpu_budget > 0 else None)
    print(json.dumps(result), flush=True)


def calibrate_copy(torch, mib: int, steps: int, warmup: int) -> None:
    """A plain copy of `mib` MiB: reads and writes `mib` MiB per launch."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: dst.copy_(src), warmup, SETTLE_MS)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        dst.copy_(src)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": steps,
                      "ms_per_copy": round(ms, 6),
                      "gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


if __name__ == "__main__":
    main()
