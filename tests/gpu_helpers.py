"""Helpers shared by the GPU tests: move seeded host inputs to the device,
run the library through its C-ABI (via the thin binding), and compare the
results with the oracle under the parity rules:

 - xOut bit-exact;
 - scales within 2e-6 relative (exactly 0 where the oracle's is 0);
 - codes equal, or off by one only where the oracle's pre-rounding value
   lies within 1e-3 of a .5 boundary; INT4 bytes are unpacked with the
   documented nibble order first.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import int4_dynamic_quantization_amd as adq
import oracle
from helpers import check_codes, check_scales, unpack_int4

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def dev(bits: np.ndarray | None, dtype: str):
    """uint16 storage patterns -> device tensor of the 16-bit type."""
    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to("cuda")


def host_bits(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def workspace(ex, fill=None):
    """Workspace for an executor: uninitialised memory by default (the
    split-row path needs no clearing), or filled with a byte value."""
    if not ex.workspace_size:
        return None
    ws = torch.empty(ex.workspace_size, dtype=torch.uint8, device="cuda")
    if fill is not None:
        ws.fill_(fill)
    return ws


def run_v2(x1, x2, g, b, s1, s2, eps, mask, y_types, dtype, path=adq.PATH_AUTO, stream=None,
           outputs=None, ws_fill=None):
    """Run AddRmsNormDynamicQuantV2 on host arrays; returns (outs, describe)."""
    ex, outs = adq.plan_add_rms_norm_dynamic_quant_v2(
        dev(x1, dtype), dev(x2, dtype), dev(g, dtype), dev(b, dtype), dev(s1, dtype),
        dev(s2, dtype), eps, mask, y_types[0], y_types[1], outputs=outputs, path=path)
    ws = workspace(ex, ws_fill)
    ex.run(ws, stream)
    torch.cuda.synchronize()
    desc = ex.describe()
    ex.close()
    return outs, desc


def run_rms(x, g, b, s, eps, y_type, dtype, path=adq.PATH_AUTO):
    ex, outs = adq.plan_rms_norm_dynamic_quant(dev(x, dtype), dev(g, dtype), dev(b, dtype),
                                               dev(s, dtype), eps, y_type, path=path)
    ws = workspace(ex)
    ex.run(ws)
    torch.cuda.synchronize()
    desc = ex.describe()
    ex.close()
    return outs, desc


def codes_of(t, qtype: str) -> np.ndarray:
    a = host(t)
    return unpack_int4(a) if qtype == "int4" else a.astype(np.int8)


def host_outputs(outs, y_types):
    """Every output of a V2 call copied to the host once: xOut storage bits,
    unpacked codes and scales (None for an output that was not produced)."""
    h = {"x_out": host_bits(outs["x_out"])}
    for k in (1, 2):
        y = outs.get(f"y{k}")
        h[f"y{k}"] = None if y is None else codes_of(y, y_types[k - 1]).reshape(y.shape[0], -1)
        sc = outs.get(f"scale{k}")
        h[f"scale{k}"] = None if sc is None else host(sc).reshape(-1)
    return h


def compare_host_v2(h, ora, r0, r1):
    """Parity of rows [r0, r1) of host copies of the outputs (host_outputs)
    with the oracle's results for those rows.  Returns the number of
    off-by-one codes at near ties."""
    assert np.array_equal(h["x_out"][r0:r1], ora["x_out"]), "xOut not bit-exact"
    ties = 0
    for k in (1, 2):
        if not ora["active"][k - 1]:
            continue
        check_scales(h[f"scale{k}"][r0:r1], ora[f"scale{k}"])
        ties += check_codes(h[f"y{k}"][r0:r1], ora[f"code{k}"], ora[f"pre{k}"])
    return ties


def oracle_v2_threaded(x1, x2, g, b, s1, s2, eps, mask, y_types, dtype, r0, r1, threads=16):
    """The oracle on rows [r0, r1), cut into contiguous parts run on host
    threads at once (its C calls release the GIL); the parts' results are
    joined in row order, so the result equals one call over the rows."""
    from concurrent.futures import ThreadPoolExecutor
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(threads, cores, r1 - r0))
    cuts = [r0 + (r1 - r0) * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(threads) as pool:
        parts = list(pool.map(
            lambda i: oracle_v2(x1[cuts[i]:cuts[i + 1]], x2[cuts[i]:cuts[i + 1]], g, b, s1, s2,
                                eps, mask, y_types, dtype), range(threads)))
    res = {"active": parts[0]["active"],
           "x_out": np.concatenate([p["x_out"] for p in parts])}
    for k in (1, 2):
        if res["active"][k - 1]:
            for key in (f"code{k}", f"scale{k}", f"pre{k}"):
                res[key] = np.concatenate([p[key] for p in parts])
    return res


def compare_v2(outs, ora, y_types, rows=None):
    """Parity of GPU outputs (optionally only `rows`) with oracle results.
    Returns the number of off-by-one codes at near ties."""
    sel = slice(None) if rows is None else rows
    assert np.array_equal(host_bits(outs["x_out"])[sel], ora["x_out"]), "xOut not bit-exact"
    ties = 0
    for k in (1, 2):
        if not ora["active"][k - 1]:
            continue
        check_scales(host(outs[f"scale{k}"]).reshape(-1)[sel], ora[f"scale{k}"])
        got = codes_of(outs[f"y{k}"], y_types[k - 1]).reshape(-1, ora[f"code{k}"].shape[1])[sel]
        ties += check_codes(got, ora[f"code{k}"], ora[f"pre{k}"])
    return ties


def compare_rms(outs, ora, y_type):
    check_scales(host(outs["scale"]).reshape(-1), ora["scale"])
    got = codes_of(outs["y"], y_type).reshape(ora["code"].shape)
    return check_codes(got, ora["code"], ora["pre"])


def oracle_v2(x1, x2, g, b, s1, s2, eps, mask, y_types, dtype, want_pre=True):
    return oracle.add_rms_norm_dq_v2(x1, x2, g, b, s1, s2, eps, mask, y_types[0], y_types[1],
                                     dtype, want_pre=want_pre)
