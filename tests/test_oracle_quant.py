"""Pins of the oracle's scale and quantise steps: exact rational arithmetic
for the float32 quotient, exact round trips, and the pages' size claim."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import e4m3, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_kv_capacity.json")


def _round_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (ties-to-even) float32 of an exact rational, for
    normal-range values: pick between the two float32 neighbours."""
    f = np.float32(float(fr))  # within an ulp
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0] or (d == best[0] and (int(c.view(np.uint32)) & 1) == 0):
            best = (d, c)
    return best[1]


def test_scale_from_amax_exact_cases():
    assert quant.scale_from_amax(448.0) == np.float32(1.0)
    assert quant.scale_from_amax(896.0) == np.float32(2.0)
    assert quant.scale_from_amax(0.0) == np.float32(1.0)
    assert quant.scale_from_amax(4.90625) == _round_f32(Fraction(4.90625) / 448)
    for a in [1.0, 3.0, 80.5, 1e-3, 7.25]:
        assert quant.scale_from_amax(a) == _round_f32(Fraction(a) / 448)


def test_quotient_is_correctly_rounded_float32_division():
    rng = np.random.default_rng(3)
    bits = (rng.integers(0, 65536, size=3000, dtype=np.uint32) << 16)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) > 1e-30) & (np.abs(x) < 1e30)]
    for s in [np.float32(4.90625 / 448), np.float32(3.0), np.float32(1.0 / 3.0)]:
        q = quant.quotient(x, s)
        for xi, qi in zip(x[:1500], q[:1500]):
            assert qi == _round_f32(Fraction(float(xi)) / Fraction(float(s)))


def test_quantize_dequantize_round_trip_on_grid():
    """fl32(code value * s) lies within a float32 ulp of a grid point, far
    inside half a code step, so it quantises back to the same code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for s in [np.float32(5.0 / 448), np.float32(1.0), np.float32(0.37)]:
        x = (e4m3.DECODE[codes] * np.float64(s)).astype(np.float32)
        assert np.array_equal(quant.quantize(x, s), codes)


def test_quantization_error_bound():
    """Within range, |dequant(quant(x)) - x| <= half a code step times s."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal(100_000).astype(np.float32)
    s = quant.scale_from_amax(float(np.abs(x).max()))
    c = quant.quantize(x, s)
    xr = quant.dequantize(c, s)
    a = np.abs(x.astype(np.float64)) / np.float64(s)
    ex = np.floor(np.log2(np.maximum(a, 2.0**-6)))
    ulp = 2.0 ** (ex - 3)
    assert np.all(np.abs(xr - x) <= 0.5 * ulp * np.float64(s) * (1 + 1e-12))


def test_fp8_pool_is_half_the_bf16_pool():
    """'halves its size' / 'twice as much' context at equal memory."""
    g = json.load(open(GOLDEN))
    per_token = lambda e: 2 * 8 * 128 * e  # K and V, 8 kv heads, head dim 128
    b16 = per_token(g["bytes_per_element"]["bf16"])
    f8 = per_token(g["bytes_per_element"]["fp8_e4m3"])
    assert b16 == 2 * f8
    budget = 686_000 * b16
    tokens_fp8 = budget // f8
    assert tokens_fp8 == 2 * 686_000
    # the pages' own rounded figures agree with an exact doubling to 0.2%
    r = g["tokens_held"]["fp8_e4m3"] / g["tokens_held"]["bf16"]
    assert abs(r - g["stated_ratio"]) < 0.005


# ---- scales set at append, one per row


def test_row_scale_puts_each_rows_largest_value_at_448():
    """The largest magnitude of every row encodes to +-448 (code 0x7E / 0xFE),
    whatever the row's range: the per-row rule always uses the full code range."""
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((50, 128)) * np.logspace(-6, 4, 50)[:, None]
    rows = rows.astype(np.float32).astype(np.float64)
    codes, scales = quant.quantize_rows(rows)
    for r in range(50):
        j = int(np.argmax(np.abs(rows[r])))
        assert codes[r, j] in (0x7E, 0xFE)
        assert scales[r] == quant.scale_from_amax(np.abs(rows[r]).max())


def test_row_scale_error_within_half_a_step():
    """Each value is off by at most half the e4m3 step at its magnitude, in
    units of its own row's scale (the RNE bound), never saturating."""
    rng = np.random.default_rng(4)
    rows = (rng.standard_normal((40, 64)) * rng.uniform(1e-3, 1e3, (40, 1))).astype(np.float32)
    codes, scales = quant.quantize_rows(rows)
    back = quant.dequantize_rows(codes, scales)
    y = np.abs(rows.astype(np.float64) / scales.astype(np.float64)[:, None])
    # e4m3 step at |y|: 2^(floor(log2 y) - 3) for normals, 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    step = 2.0 ** (e - 3)
    err = np.abs(back - rows) / scales.astype(np.float64)[:, None]
    assert np.all(err <= step / 2 + 1e-12)


def test_row_scale_zero_row_and_exact_grid_rows():
    codes, scales = quant.quantize_rows(np.zeros((2, 16)))
    assert np.all(codes == 0) and np.all(scales == 1.0)
    # a row whose values are table values times a power of two round-trips
    vals = e4m3.decode(np.array([0x7E, 0x01, 0x38, 0xC0, 0x00, 0x22], dtype=np.uint8))
    row = vals * 2.0 ** -7
    c, s = quant.quantize_rows(row[None, :])
    assert np.array_equal(quant.dequantize_rows(c, s)[0], row)


def test_row_scale_leaves_nan_out_of_the_row_amax():
    """A NaN takes no part in its row's largest magnitude and becomes a NaN
    code with its sign; the rest of the row is encoded as if it were absent.
    An all-NaN row gets scale 1 (no magnitude, as an all-zero row)."""
    row = np.array([np.nan, 224.0, -112.0, 1.0, -np.nan, 0.0], dtype=np.float64)
    c, s = quant.quantize_rows(row[None, :])
    assert s[0] == np.float32(0.5)  # 224 / 448
    assert c[0, 0] == 0x7F and c[0, 4] == 0xFF
    assert c[0, 1] == 0x7E and c[0, 2] == 0xF6 and c[0, 3] == 0x40 and c[0, 5] == 0x00
    c2, s2 = quant.quantize_rows(np.full((1, 4), np.nan))
    assert s2[0] == 1.0 and np.all(c2 == 0x7F)
    # an infinity is a magnitude: scale inf, finite values encode as zero codes and
    # inf / inf is the default NaN with the sign bit set, for either sign of inf
    c3, s3 = quant.quantize_rows(np.array([[np.inf, 3.0, -3.0, -np.inf]]))
    assert np.isinf(s3[0]) and c3[0, 0] == 0xFF and c3[0, 1] == 0x00 and c3[0, 2] == 0x80
    assert c3[0, 3] == 0xFF


def test_scale_from_amax_subnormal_results():
    """Scales that land among float32 subnormals (multiples of 2^-149) still
    round to nearest: the smallest bf16 magnitude 2^-133 gives
    2^-133 / 448 = 2^-139 / 7 = (1024 / 7) * 2^-149 = 146.29 * 2^-149, so
    s = 146 * 2^-149; and the amax value itself then sits at
    2^16 / 146 = 448.9 scale units, above 448, so it saturates to 0x7E."""
    tiny = 2.0 ** -133
    s = quant.scale_from_amax(tiny)
    assert s == np.float32(146 * 2.0 ** -149)
    assert quant.quantize(np.array([tiny, -tiny]), s).tolist() == [0x7E, 0xFE]
    # a float32-normal but small amax: 2^-100 / 448 = 2^-106 / 7, normal
    assert quant.scale_from_amax(2.0 ** -100) == _round_f32(Fraction(2) ** -100 / 448)
