"""Single-token decode attention over a paged cache, float64 reference.

"Smaller, faster, safer", section "Quantizing the KV cache": the FP8 attention
kernel converts cached values as it reads them; apart from that conversion
the decode computes ordinary softmax attention of the new token's query over
every cached key and value of its request. Section "Protecting a shared KV
cache": many requests read pages of one physical cache (paged attention).

This module is the plain definition, unsplit:
  s_t = sm_scale * sum_d q[d] * k_t[d]
  w_t = exp(s_t - max s) / sum_u exp(s_u - max s)
  o   = sum_t w_t * v_t,     lse = max s + ln sum_u exp(s_u - max s)
with query head h reading kv head h // (Hq / Hkv) (grouped-query attention;
Hq = Hkv is plain multi-head attention).

Pool layout read by ``gather``: [num_pages][Hkv][page_size][D]; token t of a
request lives in page block_table[t // P], row t % P.
"""
from __future__ import annotations

import numpy as np


def gather(pool, block_table_row, seq_len: int, page_size: int) -> np.ndarray:
    """Contiguous [L, Hkv, D] rows of one request from a paged pool."""
    pool = np.asarray(pool)
    t = np.arange(seq_len)
    pages = np.asarray(block_table_row)[t // page_size]
    rows = t % page_size
    return pool[pages, :, rows, :]


def attend(q, k, v, sm_scale: float):
    """Decode attention of one request.

    q: [Hq, Dk]; k: [L, Hkv, Dk]; v: [L, Hkv, Dv] (all float64, dequantised).
    Returns (o [Hq, Dv], lse [Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq = q.shape[0]
    hkv = k.shape[1]
    g = hq // hkv
    o = np.zeros((hq, v.shape[2]), dtype=np.float64)
    lse = np.zeros(hq, dtype=np.float64)
    for h in range(hq):
        kh = k[:, h // g, :]
        vh = v[:, h // g, :]
        s = sm_scale * (kh @ q[h])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[h] = (e / l) @ vh
        lse[h] = m + np.log(l)
    return o, lse


def weights(q, k, sm_scale: float) -> np.ndarray:
    """Softmax weights [Hq, L] (diagnostic: they sum to one per head)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    g = q.shape[0] // k.shape[1]
    out = []
    for h in range(q.shape[0]):
        s = sm_scale * (k[:, h // g, :] @ q[h])
        e = np.exp(s - s.max())
        out.append(e / e.sum())
    return np.stack(out)


def attend_drafts(q, k, v, sm_scale: float):
    """Decode attention of a request whose last T cached tokens are the current
    token and its T - 1 draft tokens, verified together (speculative decoding).

    Cloudflare's post on the infrastructure for serving extra-large models
    (its speculative decoding section) has a small draft model propose a few
    future tokens that the target model accepts or rejects in one forward
    pass; in that pass the drafts go through attention together.
    Each query position sees the context up to and including itself and no
    later draft (causal among the drafts): query j (0 <= j < T), the token at
    position L - T + j, attends to cached tokens 0 .. L - T + j.

    q: [T, Hq, Dk]; k: [L, Hkv, Dk]; v: [L, Hkv, Dv] (float64, dequantised).
    Returns (o [T, Hq, Dv], lse [T, Hq]); a query that sees no token (L < T
    leaves the first ones without any) gets o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, hq = q.shape[0], q.shape[1]
    L = k.shape[0]
    o = np.zeros((T, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((T, hq), -np.inf, dtype=np.float64)
    for j in range(T):
        n = L - T + j + 1
        if n <= 0:
            continue
        o[j], lse[j] = attend(q[j], k[:n], v[:n], sm_scale)
    return o, lse
