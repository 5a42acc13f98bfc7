"""Pins of the oracle's E4M3 codec against things other than itself:
the OCP special values (golden fixture), torch's float8_e4m3fn type (a
library implementation of the same OCP format), a brute-force nearest
search and an independent integer bit-manipulation encoder."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_special_values.json")


def test_special_values_match_ocp_table():
    g = json.load(open(GOLDEN))
    for item in g["values"]:
        c = int(item["code"], 16)
        v = e4m3.DECODE[c]
        if item["value"] == "nan":
            assert np.isnan(v), hex(c)
        else:
            assert v == item["value"], hex(c)
            assert np.signbit(v) == np.signbit(item["value"]), hex(c)
    finite = e4m3.DECODE[~np.isnan(e4m3.DECODE)]
    assert int(np.isnan(e4m3.DECODE).sum()) == g["counts"]["nan_codes"]
    assert int((finite > 0).sum()) == g["counts"]["positive_finite_nonzero"]
    assert int(np.isinf(e4m3.DECODE).sum()) == g["counts"]["infinities"]


def test_decode_matches_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(ours[ok]))


def test_decode_monotone_and_symmetric():
    pos = e4m3.DECODE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(e4m3.DECODE[0x80:0xFF], -pos)


def test_round_trip_every_non_nan_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = e4m3.encode(e4m3.DECODE[codes].astype(np.float32))
    assert np.array_equal(back, codes)


# ------------------------------------------------------------------ brute force
def _brute(y: float) -> int:
    """argmin over finite codes of |y - value|, ties to the even code;
    saturating; NaN -> NaN code with the sign of y."""
    neg = bool(np.signbit(np.float32(y)))
    if np.isnan(y):
        return 0x7F | (0x80 if neg else 0)
    a = abs(float(y))
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(a - e4m3.DECODE[c])
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    if a >= 448.0:
        best = 0x7E
    return best | (0x80 if neg else 0)


def _midpoints():
    mags = e4m3.DECODE[:0x7F].astype(np.float32)
    mids = ((mags[:-1].astype(np.float64) + mags[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    extra = np.array([0.0, 2.0**-10, 2.0**-11, 447.9, 448.0, 449.0, 464.0, 465.0, 1e30,
                      np.inf, np.nan, 1e-40, 3 * 2.0**-11], dtype=np.float32)
    vals = np.concatenate([mids, up, dn, mags, extra])
    return np.concatenate([vals, -vals])


def test_encoder_matches_brute_force_on_ties_and_neighbours():
    ys = _midpoints()
    got = e4m3.encode(ys)
    exp = np.array([_brute(y) for y in ys], dtype=np.uint8)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(float(ys[i]), hex(got[i]), hex(exp[i])) for i in bad[:10]]


# ------------------------------------------------------- independent bit encoder
def _bit_encode(y: np.ndarray) -> np.ndarray:
    """Integer RNE float32 -> E4M3 written from the IEEE bit layout."""
    y = np.asarray(y, dtype=np.float32)
    u = y.view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1) << 7
    a = u & 0x7FFFFFFF
    out = np.zeros(y.shape, dtype=np.int64)
    is_nan = a > 0x7F800000
    sat = ~is_nan & (a >= 0x43E00000)  # 448.0f
    e = (a >> 23) - 127
    man = a & 0x7FFFFF
    normal = ~is_nan & ~sat & (e >= -6)
    sub = ~is_nan & ~sat & (e < -6)
    # normal range: keep 3 of 23 mantissa bits, round half to even
    code = ((e + 7) << 3) | (man >> 20)
    rem = man & 0xFFFFF
    up = (rem > 0x80000) | ((rem == 0x80000) & ((code & 1) == 1))
    code = code + up
    out = np.where(normal, code, out)
    # below 2**-6: multiples of 2**-9, round half to even on the integer count
    scaled = np.abs(y.astype(np.float64)) * 512.0
    out = np.where(sub, np.rint(scaled).astype(np.int64), out)
    out = np.where(sat, 0x7E, out)
    out = np.where(is_nan, 0x7F, out)
    return (out | sign).astype(np.uint8)


def test_encoder_matches_bit_encoder_all_bf16_patterns_and_scales():
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    for s in [1.0, 4.90625 / 448, 5.0 / 448, 96.0 / 448, 2.0**-7, 3.0]:
        s32 = np.float32(s)
        y = (x.astype(np.float64) / np.float64(s32)).astype(np.float32)
        assert np.array_equal(e4m3.encode(y), _bit_encode(y)), s


def test_encoder_matches_bit_encoder_random_float32():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    y = u.view(np.float32)
    assert np.array_equal(e4m3.encode(y), _bit_encode(y))
    z = rng.standard_normal(200_000).astype(np.float32) * np.float32(60)
    assert np.array_equal(e4m3.encode(z), _bit_encode(z))


def test_encoder_agrees_with_torch_cast_in_range():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest even; above
    the range it does not saturate, so compare only |y| < 448."""
    rng = np.random.default_rng(9)
    y = np.concatenate([
        (rng.standard_normal(300_000) * 100).astype(np.float32),
        (rng.standard_normal(100_000) * 0.01).astype(np.float32),
        _midpoints(),
    ])
    y = y[np.isfinite(y) & (np.abs(y) < 448)]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(y), ref)


def test_saturation_and_specials():
    y = np.array([448.0, 460.0, 1e6, np.inf, -np.inf, np.nan, -0.0, 0.0, -(2.0**-11)], np.float32)
    got = e4m3.encode(y)
    assert [hex(c) for c in got] == ["0x7e", "0x7e", "0x7e", "0x7e", "0xfe", "0x7f", "0x80", "0x0", "0x80"]


@pytest.mark.parametrize("mutant", ["ties_up", "no_saturate"])
def test_planted_mistakes_are_caught(mutant):
    """Plant a plausible mistake in a copy of the encoder and check that the
    brute-force pin notices."""
    ys = _midpoints()
    exp = np.array([_brute(y) for y in ys], dtype=np.uint8)
    got = e4m3.encode(ys).copy()
    if mutant == "ties_up":
        mags = e4m3.DECODE[:0x7F]
        a = np.abs(ys.astype(np.float64))
        for i, v in enumerate(a):
            j = np.searchsorted(mags, v)
            if 0 < j < 0x7F and v == (mags[j - 1] + mags[j]) / 2:
                got[i] = (got[i] & 0x80) | j
    else:
        got[np.abs(ys) >= 448] = 0x7F | (got[np.abs(ys) >= 448] & 0x80)
    assert np.any(got != exp)
