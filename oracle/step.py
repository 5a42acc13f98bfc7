"""One decode step of a workload, computed request by request in float64.

Order of a step (reading of "Smaller, faster, safer", section "Protecting a
shared KV cache": the mapping check runs before the decode reads the cache):
  1. tag check -> per-request abort flags;
  2. every K/V value of a request is quantised with its tensor's (or kv
     head's) static scale (section "Quantizing the KV cache"): the scale is
     fl32(amax / 448) of the K (or V) values, of the whole cache or of one
     kv head;
  3. decode attention over the dequantised values, query head h reading kv
     head h // G (G = Hq / Hkv); an aborted request reads nothing and its
     output is zero (lse = -inf).
The latent layout has one row per token whose first head_dim_v values are
also V, under the one scale of that row's tensor.

Inputs come from the workload as raw bf16 bit patterns (NumPy uint16),
widened here to float64 exactly; nothing here comes from the GPU path.
A workload is any object with the attributes and methods used below
(``tests/test_oracle_step.py`` drives a hand-built one).
"""
from __future__ import annotations

import numpy as np

from . import attention, quant, verify as _verify

FP8 = "fp8"
BF16 = "bf16"


def bf16_bits_to_f64(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns: a bf16 value is the float32 whose
    upper 16 bits are the pattern and whose lower 16 bits are zero."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def scales(w, kv_dtype: str = FP8):
    """(k_scale, v_scale) float32 [Hkv]; ones for a BF16 cache. The latent
    layout's V is part of the K row and shares its scale."""
    H = w.num_kv_heads
    if kv_dtype == BF16:
        one = np.ones(H, dtype=np.float32)
        return one, one.copy()
    if w.per_head_scales:
        ks = np.array([quant.scale_from_amax(w.amax("k", h)) for h in range(H)], dtype=np.float32)
        vs = ks if w.latent else np.array(
            [quant.scale_from_amax(w.amax("v", h)) for h in range(H)], dtype=np.float32)
    else:
        ks = np.full(H, quant.scale_from_amax(w.amax("k")), dtype=np.float32)
        vs = ks if w.latent else np.full(H, quant.scale_from_amax(w.amax("v")), dtype=np.float32)
    return ks, vs.copy()


def flags(w) -> np.ndarray:
    return _verify.verify(w.page_tags, w.block_table, w.expected_tags, w.seq_lens, w.page_size)


def request_codes(w, b: int, k_scale, v_scale, heads=None, tokens=None):
    """e4m3 codes of request b's K rows (and V rows, None if latent):
    uint8 [L, nh, D] for the selected kv heads and tokens, each kv head under
    its own scale."""
    hs = np.arange(w.num_kv_heads) if heads is None else np.asarray(heads)
    x = bf16_bits_to_f64(w.k_bits(b, heads=hs, tokens=tokens))
    kc = np.stack([quant.quantize(x[:, i, :], k_scale[h]) for i, h in enumerate(hs)], axis=1)
    if w.latent:
        return kc, None
    y = bf16_bits_to_f64(w.v_bits(b, heads=hs, tokens=tokens))
    vc = np.stack([quant.quantize(y[:, i, :], v_scale[h]) for i, h in enumerate(hs)], axis=1)
    return kc, vc


def request_kv(w, b: int, kv_dtype: str, k_scale, v_scale, heads=None):
    """Dequantised float64 K [L, nh, Dk] and V [L, nh, Dv] of request b
    (a BF16 cache holds the values themselves)."""
    hs = np.arange(w.num_kv_heads) if heads is None else np.asarray(heads)
    if kv_dtype == BF16:
        k = bf16_bits_to_f64(w.k_bits(b, heads=hs))
        v = k[..., : w.head_dim_v] if w.latent else bf16_bits_to_f64(w.v_bits(b, heads=hs))
        return k, v
    kc, vc = request_codes(w, b, k_scale, v_scale, heads=hs)
    k = np.stack([quant.dequantize(kc[:, i, :], k_scale[h]) for i, h in enumerate(hs)], axis=1)
    if w.latent:
        return k, k[..., : w.head_dim_v]
    v = np.stack([quant.dequantize(vc[:, i, :], v_scale[h]) for i, h in enumerate(hs)], axis=1)
    return k, v


def request_output(w, b: int, kv_dtype: str, k_scale, v_scale, aborted: bool,
                   kv_heads=None, q=None):
    """(o [nq, Dv], lse [nq]) for the q heads of the selected kv heads of
    request b, in head order (kv head g serves q heads g G .. g G + G - 1);
    zeros and -inf if the request is aborted. q: float64 [Hq, Dk] of request
    b, or None to take the workload's."""
    G = w.group
    hs = np.arange(w.num_kv_heads) if kv_heads is None else np.asarray(kv_heads)
    qh = np.concatenate([np.arange(h * G, (h + 1) * G) for h in hs])
    if aborted:
        return (np.zeros((qh.size, w.head_dim_v)), np.full(qh.size, -np.inf))
    if q is None:
        q = bf16_bits_to_f64(w.q_bits()[b])
    k, v = request_kv(w, b, kv_dtype, k_scale, v_scale, heads=hs)
    return attention.attend(np.asarray(q, dtype=np.float64)[qh], k, v, w.sm_scale)


def run(w, kv_dtype: str = FP8, requests=None, kv_heads=None):
    """Whole step for the selected requests: dict with scales, flags, and
    per-request (o, lse)."""
    ks, vs = scales(w, kv_dtype)
    fl = flags(w)
    qall = bf16_bits_to_f64(w.q_bits())
    reqs = range(w.batch) if requests is None else requests
    outs = {}
    for b in reqs:
        outs[int(b)] = request_output(w, int(b), kv_dtype, ks, vs, bool(fl[b]), kv_heads, qall[b])
    return {"k_scale": ks, "v_scale": vs, "flags": fl, "out": outs}
