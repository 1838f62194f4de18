"""Pins of the AddLora oracle against things other than itself.

 - a hand-worked example from the Formulas of "aclnnAddLora"
   (tests/golden/lora_worked.json), with and without weightA, including
   rows outside [0, W), decoy layers and bf16 ties;
 - numpy's float64 matrix products, group by group (a library routine the
   oracle does not use), on random bf16 and fp16 data;
 - closed forms: scale 0 leaves y unchanged; identity expand weights give
   y + scale * x; rows with no adapter are copied;
 - invariants: permuting rows permutes the output; columns outside the
   slice are copied bit for bit; the stored value is the slice value
   rounded once (rounding itself is pinned in test_oracle_pins.py).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import from_bits, to_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lora_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_lora_worked_example():
    g = _golden()
    dt = g["dtype"]
    out, pre = oracle.add_lora(to_bits(g["y"], dt), to_bits(g["x"], dt), to_bits(g["weight_b"], dt),
                               np.array(g["indices"], np.int32), to_bits(g["weight_a"], dt),
                               g["layer"], g["scale"], g["y_offset"], dt)
    assert np.array_equal(from_bits(out, dt), np.array(g["out"], np.float64))
    assert np.array_equal(pre, np.array(g["pre"], np.float64))


def test_lora_worked_example_without_weight_a():
    g = _golden()
    dt = g["dtype"]
    out, _ = oracle.add_lora(to_bits(g["y"], dt), to_bits(g["x"], dt), to_bits(g["weight_b"], dt),
                             np.array(g["indices"], np.int32), None, g["layer"], g["scale"],
                             g["y_offset"], dt)
    assert np.array_equal(from_bits(out, dt), np.array(g["without_weight_a"]["out"], np.float64))


def _numpy_reference(y, x, wa, wb, idx, layer, scale, off, dt):
    """Slice values before rounding, from numpy float64 products per group."""
    yv, xv = from_bits(y, dt), from_bits(x, dt)
    w, _, rank, h2 = wb.shape
    ref = yv[:, off:off + h2].copy()
    s = float(np.float32(scale))
    for g in range(w):
        rows = np.nonzero(idx == g)[0]
        if rows.size == 0:
            continue
        z1 = xv[rows] if wa is None else xv[rows] @ from_bits(wa[g, layer], dt)
        ref[rows] += (z1 @ from_bits(wb[g, layer], dt)) * s
    mag = np.zeros_like(ref)
    for g in range(w):
        rows = np.nonzero(idx == g)[0]
        if rows.size:
            z1 = np.abs(xv[rows]) if wa is None else np.abs(xv[rows]) @ np.abs(
                from_bits(wa[g, layer], dt))
            mag[rows] = (z1 @ np.abs(from_bits(wb[g, layer], dt))) * abs(s)
    return ref, mag + np.abs(yv[:, off:off + h2])


@pytest.mark.parametrize("dt,has_a", [("bf16", True), ("fp16", True), ("bf16", False)])
def test_lora_matches_numpy_products(dt, has_a):
    # scale 0.1 is not a float: it is applied as the nearest float
    wl = synth.LoraWorkload("t", 96, 64 if has_a else 16, 16, 48, 80, 4, 3, 1, 20, 0.1, dt, 31,
                            -1, 4, has_a)
    y, x, wa, wb, idx = synth.lora_inputs(wl)
    out, pre = oracle.add_lora(y, x, wb, idx, wa, wl.layer, wl.scale, wl.y_offset, dt)
    ref, mag = _numpy_reference(y, x, wa, wb, idx, wl.layer, wl.scale, wl.y_offset, dt)
    # both sides are double sums of the same exact products, in different orders
    assert np.all(np.abs(pre - ref) <= 1e-13 * mag)
    # and the stored slice is the slice value rounded once
    rounded = np.array([oracle.round_to_storage(v, dt) for v in pre.ravel()], np.uint16)
    assert np.array_equal(out[:, wl.y_offset:wl.y_offset + wl.h2].ravel(), rounded)


def test_lora_columns_outside_slice_and_unassigned_rows_are_copied():
    wl = synth.LORA_WORKLOADS["lora_small"]
    y, x, wa, wb, idx = synth.lora_inputs(wl)
    out, _ = oracle.add_lora(y, x, wb, idx, wa, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    keep = np.ones(wl.h3, bool)
    keep[wl.y_offset:wl.y_offset + wl.h2] = False
    assert np.array_equal(out[:, keep], y[:, keep])
    none = (idx < 0) | (idx >= wl.w)
    assert none.any() and np.array_equal(out[none], y[none])
    assert not np.array_equal(out[~none], y[~none])


def test_lora_scale_zero_is_identity():
    wl = synth.LORA_WORKLOADS["lora_small"]
    y, x, wa, wb, idx = synth.lora_inputs(wl, rows=64)
    out, _ = oracle.add_lora(y, x, wb, idx, wa, wl.layer, 0.0, wl.y_offset, wl.dtype)
    assert np.array_equal(out, y)


def test_lora_identity_expand_closed_form():
    """No weightA and B[g, layer] = identity (rank = h2): out = y + scale * x
    on the slice, for every adapter."""
    rows, h, h3, w, layers, off, scale = 40, 16, 24, 3, 2, 5, 0.375
    wl = synth.LoraWorkload("t", rows, h, h, h, h3, w, layers, 1, off, scale, "bf16", 5)
    y, x, _, _, idx = synth.lora_inputs(wl)
    wb = np.zeros((w, layers, h, h), np.uint16)
    wb[:, 1] = to_bits(np.eye(h), "bf16")
    wb[:, 0] = to_bits(np.full((h, h), 3.0), "bf16")  # decoy layer
    _, pre = oracle.add_lora(y, x, wb, idx, None, 1, scale, off, "bf16")
    expect = from_bits(y, "bf16")[:, off:off + h] + scale * from_bits(x, "bf16")
    assert np.array_equal(pre, expect)


def test_lora_row_permutation():
    wl = synth.LORA_WORKLOADS["lora_small"]
    y, x, wa, wb, idx = synth.lora_inputs(wl, rows=80)
    perm = np.random.default_rng(3).permutation(80)
    out, _ = oracle.add_lora(y, x, wb, idx, wa, wl.layer, wl.scale, wl.y_offset, wl.dtype)
    outp, _ = oracle.add_lora(y[perm], x[perm], wb, idx[perm], wa, wl.layer, wl.scale,
                              wl.y_offset, wl.dtype)
    assert np.array_equal(outp, out[perm])
    # and a subset of rows gives the same rows
    sub, _ = oracle.add_lora(y, x, wb, idx, wa, wl.layer, wl.scale, wl.y_offset, wl.dtype,
                             rows=perm[:10])
    assert np.array_equal(sub, out[perm[:10]])


def test_lora_rejects_bad_arguments():
    g = _golden()
    dt = g["dtype"]
    args = (to_bits(g["y"], dt), to_bits(g["x"], dt), to_bits(g["weight_b"], dt),
            np.array(g["indices"], np.int32), to_bits(g["weight_a"], dt))
    with pytest.raises(ValueError):
        oracle.add_lora(*args, layer=2, scale=1.0, y_offset=0, dtype=dt)   # layer out of range
    with pytest.raises(ValueError):
        oracle.add_lora(*args, layer=1, scale=1.0, y_offset=3, dtype=dt)   # slice past h3
