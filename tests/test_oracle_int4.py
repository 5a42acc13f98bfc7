"""Pins of the INT4 linear-layer oracle (oracle/int4.py) against hand-decoded
nibbles, a hand-worked layer (tests/golden/), the bijection between bytes
and code pairs, the placement of group scales, and a brute force."""
import json
import math
import os

import numpy as np

import workloads as W
from oracle import int4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_unpack_matches_hand_decoded_bytes():
    g = json.load(open(os.path.join(GOLD, "int4_nibbles.json")))
    for e in g["bytes"]:
        codes = int4.unpack(np.array([[int(e["byte"], 16)]], dtype=np.uint8))
        assert codes.tolist() == [[e["even_k"], e["odd_k"]]], e


def test_bytes_and_code_pairs_are_a_bijection():
    """The 256 bytes decode to the 256 pairs of [-8, 7] x [-8, 7], each once."""
    codes = int4.unpack(np.arange(256, dtype=np.uint8).reshape(256, 1))
    pairs = {tuple(r) for r in codes.tolist()}
    assert len(pairs) == 256
    assert all(-8 <= a <= 7 and -8 <= b <= 7 for a, b in pairs)


def test_hand_worked_layer():
    g = json.load(open(os.path.join(GOLD, "int4_layer_example.json")))
    n, k = g["n"], g["k"]
    packed = np.array([[int(b, 16)] * (k // 2) for b in g["row_bytes"]], dtype=np.uint8)
    scales = np.array(g["scales_group_major"], dtype=np.float64)  # [group][n]
    x = np.zeros((2, k))
    x[0, :128], x[0, 128:] = 1.0, 2.0
    x[1, 129] = 1.0
    y = int4.linear(x, packed, scales, g["group"])
    assert np.array_equal(y, np.array(g["y"]))


def test_group_scale_placement():
    """Codes of 1 everywhere: each weight is its own (row, group) scale, and a
    scale reaches exactly the 128 inputs of its group."""
    n, k = 3, 512
    packed = np.full((n, k // 2), 0x11, dtype=np.uint8)
    scales = (np.arange(4 * n, dtype=np.float64).reshape(4, n) + 1.0) / 8.0
    w = int4.dequantize(packed, scales)
    for r in range(n):
        for kk in (0, 127, 128, 255, 256, 511):
            assert w[r, kk] == scales[kk // 128, r]
    neg = int4.dequantize(np.full((n, k // 2), 0x88, dtype=np.uint8), scales)
    assert np.array_equal(neg, -8.0 * w)


def test_linear_brute_force():
    """Random layer from the input generator: every output against a
    per-element sum with math.fsum, weights decoded nibble by nibble."""
    lay = W.int4_custom("bf", 7, 6, 256, 3)
    packed = lay.codes().numpy()
    scales = lay.scales().float().numpy().astype(np.float64)
    x = lay.x().float().numpy().astype(np.float64)
    y = int4.linear(x, packed, scales)
    for b in range(3):
        for r in range(6):
            terms = []
            for kk in range(256):
                byte = int(packed[r, kk // 2])
                nib = (byte >> 4) if kk % 2 else (byte & 15)
                q = nib - 16 if nib > 7 else nib
                terms.append(x[b, kk] * q * scales[kk // 128, r])
            assert math.isclose(y[b, r], math.fsum(terms), rel_tol=1e-12, abs_tol=1e-12)


def test_linearity_in_x_and_scales():
    lay = W.int4_custom("lin", 8, 16, 384, 2)
    packed = lay.codes().numpy()
    scales = lay.scales().float().numpy().astype(np.float64)
    x = lay.x().float().numpy().astype(np.float64)
    y = int4.linear(x, packed, scales)
    assert np.array_equal(int4.linear(2.0 * x, packed, scales), 2.0 * y)
    assert np.array_equal(int4.linear(x, packed, 0.5 * scales), 0.5 * y)
    one_hot = np.zeros((1, 384))
    one_hot[0, 200] = 1.0
    w = int4.dequantize(packed, scales)
    assert np.array_equal(int4.linear(one_hot, packed, scales)[0], w[:, 200])
