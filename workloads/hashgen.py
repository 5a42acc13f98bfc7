"""Counter-based synthetic bf16 values, identical on CPU and GPU.

This module holds no attention or quantisation arithmetic: it only draws
inputs. Every value is a pure function of (stream key, element index):

    h   = mix32(mix32(idx ^ k0) ^ k1)
    u   = h >> 12                        (a 20-bit bucket)
    val = NORMAL_BF16[u]                 (bf16 of the standard-normal quantile
                                          at probability (u + 1/2) / 2**20)

``mix32`` is the "lowbias32" 32-bit integer hash published by Chris Wellons
("Prospecting for Hash Functions", 2018): xorshift 16, multiply 0x7feb352d,
xorshift 15, multiply 0x846ca68b, xorshift 16. It is a bijection on 32-bit
words, which is what lets ``amax_bits`` find the largest magnitudes of a
tensor by inverting it instead of scanning billions of elements.

Outliers: an element is an outlier iff
``mix32(mix32(idx ^ k2) ^ k3) < OUTLIER_THRESHOLD``; outliers take
``NORMAL_X20_BF16[u]`` (the fp32 quantile times 20, then rounded to bf16).

The same torch integer code runs on CPU and GPU, so a GPU bulk fill and a
CPU sample of the same request hold the same bits. Multiplications are done
on 16-bit halves in int64 so that nothing overflows.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

M32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x846CA68B
_C1_INV = pow(_C1, -1, 2**32)
_C2_INV = pow(_C2, -1, 2**32)

TABLE_BITS = 20
TABLE_SIZE = 1 << TABLE_BITS
_BUCKET_SHIFT = 32 - TABLE_BITS
OUTLIER_FRAC = 0.001
OUTLIER_SCALE = 20.0
OUTLIER_THRESHOLD = int(round(OUTLIER_FRAC * 2**32))


# ----------------------------------------------------------------------------
# keys
# ----------------------------------------------------------------------------
def stream_keys(seed: int, *path: int) -> tuple[int, int, int, int]:
    """Four 32-bit keys for one named stream (seed, *path), via SeedSequence."""
    st = np.random.SeedSequence([int(seed), *[int(p) for p in path]]).generate_state(4)
    return tuple(int(x) for x in st)


# ----------------------------------------------------------------------------
# bf16 rounding of the tables (input preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@functools.lru_cache(maxsize=None)
def _tables() -> tuple[np.ndarray, np.ndarray]:
    from scipy.special import ndtri

    half = TABLE_SIZE // 2
    p = (np.arange(half, dtype=np.float64) + 0.5) / TABLE_SIZE
    z_neg = ndtri(p).astype(np.float32)  # strictly increasing, all < 0
    z = np.concatenate([z_neg, -z_neg[::-1]])  # exact mirror symmetry
    n_bits = f32_to_bf16_bits(z)
    x20 = (z * np.float32(OUTLIER_SCALE)).astype(np.float32)
    o_bits = f32_to_bf16_bits(x20)
    return n_bits, o_bits


def normal_table() -> np.ndarray:
    """uint16 bf16 bits of the 2**20 normal quantiles (mirror-symmetric)."""
    return _tables()[0]


def outlier_table() -> np.ndarray:
    return _tables()[1]


_dev_tables: dict = {}


def _tables_on(device) -> tuple[torch.Tensor, torch.Tensor]:
    key = str(torch.device(device))
    if key not in _dev_tables:
        n_bits, o_bits = _tables()
        _dev_tables[key] = (
            torch.from_numpy(n_bits.view(np.int16).copy()).to(device),
            torch.from_numpy(o_bits.view(np.int16).copy()).to(device),
        )
    return _dev_tables[key]


# ----------------------------------------------------------------------------
# the hash: torch (CPU or GPU) and numpy (uint32) forms
# ----------------------------------------------------------------------------
def _mul32_t(x: torch.Tensor, c: int) -> torch.Tensor:
    return ((x * (c & 0xFFFF)) + (((x * (c >> 16)) & 0xFFFF) << 16)) & M32


def mix32_t(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 on int64 tensors holding values in [0, 2**32)."""
    x = x ^ (x >> 16)
    x = _mul32_t(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32_t(x, _C2)
    return x ^ (x >> 16)


def mix32_np(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.uint32).copy()
    x ^= x >> np.uint32(16)
    x *= np.uint32(_C1)
    x ^= x >> np.uint32(15)
    x *= np.uint32(_C2)
    x ^= x >> np.uint32(16)
    return x


def unmix32_np(h: np.ndarray) -> np.ndarray:
    """Inverse of ``mix32_np``."""
    x = np.asarray(h, dtype=np.uint32).copy()
    x ^= x >> np.uint32(16)
    x *= np.uint32(_C2_INV)
    x ^= (x >> np.uint32(15)) ^ (x >> np.uint32(30))
    x *= np.uint32(_C1_INV)
    x ^= x >> np.uint32(16)
    return x


# ----------------------------------------------------------------------------
# value generation
# ----------------------------------------------------------------------------
def bf16_from_index(keys, idx: torch.Tensor, outliers: bool = False) -> torch.Tensor:
    """bf16 values for int64 element indices ``idx`` (any shape, any device)."""
    k0, k1, k2, k3 = keys
    tab, tab20 = _tables_on(idx.device)
    h = mix32_t(mix32_t(idx ^ k0) ^ k1)
    bits = tab[h >> _BUCKET_SHIFT]
    if outliers:
        h2 = mix32_t(mix32_t(idx ^ k2) ^ k3)
        bits = torch.where(h2 < OUTLIER_THRESHOLD, tab20[h >> _BUCKET_SHIFT], bits)
    return bits.view(torch.bfloat16)


def bf16_block(keys, n: int, device="cpu", outliers: bool = False,
               chunk: int = 1 << 26) -> torch.Tensor:
    """The first ``n`` values of a stream, as a flat bf16 tensor."""
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(s, e, dtype=torch.int64, device=device)
        out[s:e] = bf16_from_index(keys, idx, outliers)
    return out


def u8_from_index(keys, idx: torch.Tensor) -> torch.Tensor:
    """Uniform bytes for int64 element indices ``idx``: the top 8 bits of
    mix32(mix32(idx ^ k0) ^ k1)."""
    k0, k1 = keys[0], keys[1]
    return (mix32_t(mix32_t(idx ^ k0) ^ k1) >> 24).to(torch.uint8)


def u8_block(keys, n: int, device="cpu", chunk: int = 1 << 26) -> torch.Tensor:
    """The first ``n`` bytes of a stream, as a flat uint8 tensor."""
    out = torch.empty(n, dtype=torch.uint8, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(s, e, dtype=torch.int64, device=device)
        out[s:e] = u8_from_index(keys, idx)
    return out


# ----------------------------------------------------------------------------
# exact max |value| of a stream prefix, by inverting the hash
# ----------------------------------------------------------------------------
def _forward_bucket_np(keys, idx: np.ndarray) -> np.ndarray:
    k0, k1 = keys[0], keys[1]
    h = mix32_np(mix32_np(idx.astype(np.uint32) ^ np.uint32(k0)) ^ np.uint32(k1))
    return (h >> np.uint32(_BUCKET_SHIFT)).astype(np.int64)


def _is_outlier_np(keys, idx: np.ndarray) -> np.ndarray:
    k2, k3 = keys[2], keys[3]
    h2 = mix32_np(mix32_np(idx.astype(np.uint32) ^ np.uint32(k2)) ^ np.uint32(k3))
    return h2 < np.uint32(OUTLIER_THRESHOLD)


def _abs_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint16) & np.uint16(0x7FFF)).astype(np.int64)


def amax_bits(keys, n: int, select=None, outliers: bool = False,
              brute_limit: int = 1 << 22) -> int:
    """Exact max over i < n (and ``select(i)`` if given) of |value_i|, as
    bf16 magnitude bits (0..0x7F80).

    Small prefixes are scanned. Large ones use the bijection: bucket u holds
    the indices mix^-1(mix^-1(h) ^ k1) ^ k0 for h in [u * 4096, (u+1) * 4096);
    the table is mirror-symmetric and its magnitude falls monotonically from
    both ends, so the first level k whose buckets {k, 2**20 - 1 - k} hold a
    selected index gives the maximum.
    """
    tab, tab20 = normal_table(), outlier_table()
    if n <= 0:
        return 0
    if n <= brute_limit:
        idx = np.arange(n, dtype=np.int64)
        if select is not None:
            idx = idx[select(idx)]
        if idx.size == 0:
            return 0
        u = _forward_bucket_np(keys, idx)
        bits = tab[u]
        if outliers:
            o = _is_outlier_np(keys, idx)
            bits = np.where(o, tab20[u], bits)
        return int(_abs_bits(bits).max())

    best = 0
    if outliers:
        # enumerate every outlier index below n through the second hash
        k2, k3 = keys[2], keys[3]
        step = 1 << 22
        for s in range(0, OUTLIER_THRESHOLD, step):
            h2 = np.arange(s, min(OUTLIER_THRESHOLD, s + step), dtype=np.uint32)
            idx = (unmix32_np(unmix32_np(h2) ^ np.uint32(k3)) ^ np.uint32(k2)).astype(np.int64)
            idx = idx[idx < n]
            if select is not None:
                idx = idx[select(idx)]
            if idx.size:
                best = max(best, int(_abs_bits(tab20[_forward_bucket_np(keys, idx)]).max()))
    k0, k1 = keys[0], keys[1]
    per_bucket = 1 << _BUCKET_SHIFT
    for level in range(TABLE_SIZE // 2):
        mag = int(_abs_bits(tab[level:level + 1])[0])
        if mag <= best:
            break
        hs = np.concatenate([
            np.arange(level * per_bucket, (level + 1) * per_bucket, dtype=np.uint64),
            np.arange((TABLE_SIZE - 1 - level) * per_bucket,
                      (TABLE_SIZE - level) * per_bucket, dtype=np.uint64),
        ]).astype(np.uint32)
        idx = (unmix32_np(unmix32_np(hs) ^ np.uint32(k1)) ^ np.uint32(k0)).astype(np.int64)
        idx = idx[idx < n]
        if select is not None and idx.size:
            idx = idx[select(idx)]
        if outliers and idx.size:
            idx = idx[~_is_outlier_np(keys, idx)]
        if idx.size:
            best = max(best, mag)
            break
    return best
