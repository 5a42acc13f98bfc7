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
    """fl32(x / s) for float32-representable x (bf16 inputs) and float32 s."""
    return (np.asarray(x, dtype=np.float64) / np.float64(np.float32(s))).astype(np.float32)


def quantize(x, s) -> np.ndarray:
    """uint8 e4m3 codes of bf16 values x under scale s."""
    return e4m3.encode(quotient(x, s))


def dequantize(codes, s) -> np.ndarray:
    """float64 value each code stands for: decode(code) * s."""
    return e4m3.decode(codes) * np.float64(np.float32(s))
