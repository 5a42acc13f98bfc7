"""INT4 weight-only linear layer of the decode phase, float64 reference.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use the oracle.

"Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare blog),
section on model weights: GLM's weights are compressed from 8-bit floating
point to 4-bit integers for decode, because producing each token streams the
weights out of GPU memory and fewer bytes make that faster; prefill expands
them back instead.

The pages give no INT4 format; the reading taken here, written out plainly:
  - a code q is a 4-bit two's-complement integer, -8 <= q <= 7;
  - two codes per byte: input k of a row sits in byte k // 2, even k in the
    low nibble (bits 0..3), odd k in the high nibble (bits 4..7);
  - one scale per (output row n, group of `group` consecutive inputs),
    stored group-major as scales[k // group][n];
  - the weight is w[n][k] = q[n][k] * scales[k // group][n];
  - the layer computes y[b][n] = sum_k x[b][k] * w[n][k].
"""
from __future__ import annotations

import numpy as np


def unpack(packed) -> np.ndarray:
    """uint8 [n][k/2] -> int8 [n][k], each nibble read as 4-bit two's complement."""
    b = np.asarray(packed, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    codes = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int16)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    codes = np.where(codes >= 8, codes - 16, codes)
    return codes.astype(np.int8)


def dequantize(packed, scales, group: int = 128) -> np.ndarray:
    """float64 weights [n][k]: code times the scale of its (row, group)."""
    q = unpack(packed).astype(np.float64)
    s = np.asarray(scales, dtype=np.float64)  # [k / group][n]
    n, k = q.shape
    assert s.shape == (k // group, n) and k % group == 0
    return q * np.repeat(s.T, group, axis=1)


def linear(x, packed, scales, group: int = 128) -> np.ndarray:
    """float64 [batch][n] = x [batch][k] @ W^T, W the dequantised weights."""
    w = dequantize(packed, scales, group)
    return np.asarray(x, dtype=np.float64) @ w.T
