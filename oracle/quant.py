"""Scales and quantise-on-append, float64 reference.

"Smaller, faster, safer", section "Quantizing the KV cache": K and V are
stored as FP8 e4m3 rather than BF16. The pages give no scale rule; the one
taken is a static per-tensor (or per K|V, kv-head) scale
s = fl32(amax / 448), with s = 1 when amax = 0, and each new value x is
stored as e4m3(fl32(x / s)).

fl32(a / b) is computed as float32(float64(a) / float64(b)): the float64
quotient of two float32 numbers rounds to float32 exactly as a correctly
rounded float32 division would (53 >= 2*24 + 2, so the double rounding is
innocuous for division).
"""
from __future__ import annotations

import numpy as np

from . import e4m3


def scale_from_amax(amax: float) -> np.float32:
    """float32 dequantisation scale for a tensor whose largest |value| is amax."""
    a = float(amax)
    if a == 0.0:
        return np.float32(1.0)
    return np.float32(np.float64(a) / np.float64(448.0))


def quotient(x, s) -> np.ndarray:
    """fl32(x / s) for float32-representable x (bf16 inputs) and float32 s.

    A NaN that the division itself creates from non-NaN operands (an infinity
    over an infinite scale) is taken as the default NaN with the sign bit
    set, whatever the signs of the operands (the GPU's divide gives it, as
    does x86 double division); an input NaN keeps its sign."""
    xa = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        q = (xa / np.float64(np.float32(s))).astype(np.float32)
    made = np.isnan(q) & ~np.isnan(xa)
    if np.any(made):
        q = np.where(made, -np.float32(np.nan), q)
    return q


def quantize(x, s) -> np.ndarray:
    """uint8 e4m3 codes of bf16 values x under scale s."""
    return e4m3.encode(quotient(x, s))


def dequantize(codes, s) -> np.ndarray:
    """float64 value each code stands for: decode(code) * s."""
    return e4m3.decode(codes) * np.float64(np.float32(s))


# ----------------------------------------------------------------------------
# Scales set at append, one per cached row
# ----------------------------------------------------------------------------
# The pages give no scale granularity. The finer reading taken here: every
# appended row (one token of one kv head, K and V separately) gets its own
# scale from its own largest magnitude, by the same rule as the static
# scales, and is encoded under it. A NaN in a row is no magnitude: it takes
# no part in the row's largest magnitude (an all-NaN row counts as all
# zero, scale 1) and is itself encoded as a NaN code, so it spoils no other
# value of its row.


def row_amax(row) -> float:
    """Largest |value| of a row, NaNs left out (0 for an empty or all-NaN row)."""
    a = np.abs(np.asarray(row, dtype=np.float64))
    a = a[~np.isnan(a)]
    return float(a.max()) if a.size else 0.0


def quantize_rows(x):
    """x: float [..., D] rows of bf16 values -> (uint8 codes [..., D],
    float32 scales [...]): scale_from_amax of each row, then quantize."""
    a = np.asarray(x, dtype=np.float64)
    flat = a.reshape(-1, a.shape[-1])
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty(flat.shape[0], dtype=np.float32)
    for i, row in enumerate(flat):
        s = scale_from_amax(row_amax(row))
        scales[i] = s
        codes[i] = quantize(row, s)
    return codes.reshape(a.shape), scales.reshape(a.shape[:-1])


def dequantize_rows(codes, scales) -> np.ndarray:
    """float64 [..., D]: decode(code) times its row's scale."""
    return e4m3.decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]
