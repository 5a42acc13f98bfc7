"""Pins of the oracle's prefill -> decode page handoff: codes of values on
the scaled e4m3 grid come back exactly, every code is within half a grid
step of its value (saturating at 448), and only the listed destination pages
and their tags change."""
import numpy as np

from oracle import e4m3, handoff


def _grid_values(rng, shape, s):
    """bf16-representable values that are exactly code * s for finite codes
    (s a power of two keeps the products exact)."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=shape)
    return codes, e4m3.DECODE[codes] * s


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(1)
    H, P, D = 2, 16, 32
    s = np.float32(0.25)
    codes, vals = _grid_values(rng, (3, H, P, D), float(s))
    dst = np.zeros((5, H, P, D), dtype=np.uint8)
    out, _ = handoff.requantize_pages(vals, dst, None, [0, 1, 2], [4, 0, 2], np.full(H, s))
    # -0 and +0 both stand for 0: compare values, and signs of zeros separately
    for sp, dp in zip([0, 1, 2], [4, 0, 2]):
        got = out[dp]
        want = codes[sp]
        same = (got == want) | ((want & 0x7F) == 0) & ((got & 0x7F) == 0) & ((got & 0x80) == (want & 0x80))
        assert np.all(same)
    assert np.all(out[1] == 0) and np.all(out[3] == 0)


def test_codes_within_half_a_grid_step():
    rng = np.random.default_rng(2)
    H, P, D = 3, 16, 64
    s = np.array([0.01, 0.5, 3.0], dtype=np.float32)
    x = rng.standard_normal((2, H, P, D)) * np.array([1.0, 50.0, 2000.0])[None, :, None, None]
    x = x.astype(np.float32).astype(np.float64)
    dst = np.zeros((2, H, P, D), dtype=np.uint8)
    out, _ = handoff.requantize_pages(x, dst, None, [0, 1], [1, 0], s)
    pos = np.sort(np.unique(e4m3.DECODE[:0x7F]))
    for sp, dp in ((0, 1), (1, 0)):
        for h in range(H):
            y = x[sp, h] / np.float64(s[h])
            val = e4m3.DECODE[out[dp, h]]
            a = np.abs(y)
            big = a >= 448.0
            assert np.all(np.abs(val[big]) == 448.0) and np.all(np.sign(val[big]) == np.sign(y[big]))
            # grid neighbours of |y| below 448
            k = np.clip(np.searchsorted(pos, a[~big]), 1, len(pos) - 1)
            step = pos[k] - pos[k - 1]
            assert np.all(np.abs(np.abs(val[~big]) - a[~big]) <= step / 2 * (1 + 1e-6) + 1e-300)


def test_only_listed_pages_and_tags_change_and_bad_pairs_are_skipped():
    rng = np.random.default_rng(3)
    H, P, D = 1, 16, 16
    x = rng.standard_normal((4, H, P, D))
    dst = rng.integers(0, 256, size=(6, H, P, D)).astype(np.uint8)
    tags = rng.integers(0, 2**32, size=6, dtype=np.uint64).astype(np.uint32)
    src_pages, dst_pages = [0, 3, -1, 2, 7], [5, 1, 2, 9, 0]
    new = np.array([11, 22, 33, 44, 55], dtype=np.uint32)
    out, t = handoff.requantize_pages(x, dst, tags, src_pages, dst_pages, np.ones(H, np.float32), new)
    for p in (0, 2, 3, 4):  # pairs (-1, 2), (2, 9) and (7, 0) name a page outside a pool
        assert np.array_equal(out[p], dst[p]) and t[p] == tags[p]
    assert t[5] == 11 and t[1] == 22
    assert not np.array_equal(out[5], dst[5])
