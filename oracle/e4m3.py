"""OCP 8-bit floating point E4M3 ("E4M3FN") codec in float64.

The pages ("Smaller, faster, safer", section "Quantizing the KV cache") name
the cache element only as "FP8, e4m3". The format taken is the OCP 8-bit
Floating Point Specification (OFP8) E4M3 encoding: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; S.1111.111 is NaN, there is no infinity;
the largest magnitude is 448 and the smallest subnormal 2**-9. (Not the
"FNUZ" variant, whose maximum is 240.)

Rounding, which the pages leave open, is round-to-nearest-even with
saturation: magnitudes at or above 448 (and infinities) become +-448, NaN
becomes the NaN code of the same sign, and the sign of zero is kept.
"""
from __future__ import annotations

import numpy as np

NAN_CODE = 0x7F
MAX_CODE = 0x7E
MAX_VALUE = 448.0


def _decode_one(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9  # subnormal: 0.mmm * 2**(1-7)
    return s * (8 + m) * 2.0 ** (e - 10)  # normal: 1.mmm * 2**(e-7)


DECODE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
DECODE.setflags(write=False)

# magnitudes of codes 0x00..0x7E, strictly increasing
_MAGS = DECODE[: MAX_CODE + 1].copy()


def decode(codes) -> np.ndarray:
    """float64 value of each uint8 code."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(y) -> np.ndarray:
    """Round float32 values to E4M3 codes (nearest, ties to even code, saturating).

    ``y`` is taken as float32 (the quotient the quantiser produces); each
    value goes to the table magnitude nearest to |y|; on a tie the code with
    a zero last mantissa bit wins, which is IEEE round-half-to-even because the
    code's lowest bit is the mantissa's lowest bit.
    """
    y32 = np.asarray(y, dtype=np.float32)
    a = np.abs(y32.astype(np.float64))
    neg = np.signbit(y32)
    out = np.empty(y32.shape, dtype=np.uint8)

    nan = np.isnan(a)
    sat = ~nan & (a >= MAX_VALUE)
    fin = ~nan & ~sat

    af = a[fin]
    hi = np.searchsorted(_MAGS, af, side="left")  # first magnitude >= af
    hi = np.minimum(hi, MAX_CODE)
    lo = np.maximum(hi - 1, 0)
    d_lo = af - _MAGS[lo]
    d_hi = _MAGS[hi] - af
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_MAGS[hi] == af, hi, code)  # exact hit
    out[fin] = code.astype(np.uint8)
    out[sat] = MAX_CODE
    out[nan] = NAN_CODE
    out |= np.where(neg, 0x80, 0).astype(np.uint8)
    return out
