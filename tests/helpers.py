"""Small test helpers: 16-bit storage conversions through numpy, and the
parity rule used to compare any implementation with the oracle.

The conversions here use numpy's own float16 and float32 types, never the
oracle's decoder, so that tests which use them check the oracle against an
independent routine.
"""
from __future__ import annotations

import numpy as np


def to_bits(values, dtype: str) -> np.ndarray:
    """Bit patterns of values that are exactly representable in dtype."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == "fp16":
        h = v.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), v, equal_nan=True), "not exact in fp16"
        return h.view(np.uint16)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v, equal_nan=True), "not exact in float"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "not exact in bf16"
    return (u >> 16).astype(np.uint16)


def from_bits(bits, dtype: str) -> np.ndarray:
    """Values of 16-bit storage patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return b.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):  # NaN patterns decode to NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def near_tie(pre: np.ndarray, tol: float = 1e-3) -> np.ndarray:
    """True where a pre-rounding value lies within tol of a .5 boundary."""
    frac = np.abs(pre) - np.floor(np.abs(pre))
    return np.abs(frac - 0.5) < tol


def check_codes(got: np.ndarray, want: np.ndarray, pre: np.ndarray, tol: float = 1e-3):
    """Codes agree exactly, except by at most 1 where the oracle's
    pre-rounding value lies within tol of a .5 boundary."""
    got = got.astype(np.int32)
    want = want.astype(np.int32)
    diff = np.abs(got - want)
    bad = (diff > 1) | ((diff == 1) & ~near_tie(pre, tol))
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), int(got[tuple(i)]), int(want[tuple(i)]), float(pre[tuple(i)]))
                  for i in idx]
        raise AssertionError(f"{int(bad.sum())} code mismatches, first: {detail}")
    return int((diff == 1).sum())


def check_scales(got: np.ndarray, want: np.ndarray, rel: float = 2e-6):
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    zero = want == 0
    assert np.all(got[zero] == 0), "scale should be exactly 0 where the row max is 0"
    err = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    if err.size and err.max() > rel:
        i = int(np.argmax(err))
        raise AssertionError(f"scale rel err {err.max():.3g} > {rel} (index {i})")
    return float(err.max()) if err.size else 0.0


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Two's complement nibbles, even column in the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo).astype(np.int8)
    hi = np.where(hi > 7, hi - 16, hi).astype(np.int8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out
