"""KV-cache integrity check, reference loop.

"Smaller, faster, safer", section "Protecting a shared KV cache": each
physical page has a tag that changes whenever it is reallocated; the server
records which pages and tags each request expects; before decode reads the
cache those mappings are checked, and a request with any mismatch is aborted
instead of reading another request's page. The check is a separate batch
pass, not part of the attention kernel.

Readings: a request reads the first ceil(L / P) entries of its block-table
row (L counts the token appended this step); a page id outside
[0, num_pages) among them is a mismatch too; entries past them are ignored.
"""
from __future__ import annotations

import numpy as np


def verify(page_tags, block_table, expected_tags, seq_lens, page_size) -> np.ndarray:
    """uint8 [B]: 1 where request b must be aborted, else 0."""
    page_tags = np.asarray(page_tags, dtype=np.uint32)
    bt = np.asarray(block_table)
    exp = np.asarray(expected_tags, dtype=np.uint32)
    lens = np.asarray(seq_lens)
    num_pages = page_tags.shape[0]
    out = np.zeros(len(lens), dtype=np.uint8)
    for b in range(len(lens)):
        n = -(-int(lens[b]) // page_size) if lens[b] > 0 else 0
        if n > bt.shape[1]:
            # tokens beyond the row have no page at all: unmapped, like an
            # id outside the pool
            out[b] = 1
            continue
        for j in range(n):
            pid = int(bt[b, j])
            if pid < 0 or pid >= num_pages or int(page_tags[pid]) != int(exp[b, j]):
                out[b] = 1
                break
    return out
