"""Prefill -> decode handoff of whole cache pages, reference (exact).

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use the oracle.

"Smaller, faster, safer", section "Quantizing the KV cache": the decode
servers hold K and V as FP8 e4m3 while the prefill side keeps BF16, so the
pages a prefill produced are re-encoded on their way into the decode pool.
Section "Protecting a shared KV cache": a page's tag changes whenever the
page is (re)allocated, and the scheduler records the tag each request
expects; a page handed to a request therefore gets a new tag.

The pages print no handoff procedure; the reading taken here: every value of
a listed source page is quantised exactly as a newly appended value would be
(quant.quantize under the destination pool's static scale of its kv head),
the destination page receives the codes in the same [kv head][row][dim]
place, its tag becomes the given new tag, and a pair naming a page outside
either pool is skipped.
"""
from __future__ import annotations

import numpy as np

from . import quant


def requantize_pages(src_pool, dst_codes, dst_tags, src_pages, dst_pages, scales, new_tags=None):
    """Returns (codes, tags) after the handoff.

    src_pool:  float64 [num_src_pages][H][P][D], the BF16 values of the source pool
    dst_codes: uint8 [num_dst_pages][H][P][D], the destination pool before
    dst_tags:  uint32 [num_dst_pages] or None
    src_pages, dst_pages: int [n], page pairs
    scales:    float32 [H], the destination pool's scales
    new_tags:  uint32 [n] or None (tags untouched)
    """
    src_pool = np.asarray(src_pool, dtype=np.float64)
    codes = np.array(dst_codes, dtype=np.uint8, copy=True)
    tags = None if dst_tags is None else np.array(dst_tags, dtype=np.uint32, copy=True)
    n_src, n_dst = src_pool.shape[0], codes.shape[0]
    for i, (sp, dp) in enumerate(zip(src_pages, dst_pages)):
        sp, dp = int(sp), int(dp)
        if not (0 <= sp < n_src and 0 <= dp < n_dst):
            continue
        for h in range(src_pool.shape[1]):
            codes[dp, h] = quant.quantize(src_pool[sp, h], scales[h])
        if new_tags is not None and tags is not None:
            tags[dp] = np.uint32(new_tags[i])
    return codes, tags
