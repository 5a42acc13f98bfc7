"""Split-KV partials and their log-sum-exp merge, float64 reference.

Not a step the pages describe: splitting a request's context into chunks of
S tokens, attending each chunk alone and merging the chunk results is a
reordering of the same softmax sum, used here for long contexts. Chunk c
covers tokens [c*S, min((c+1)*S, L)). The merge of chunk results
(o_c, lse_c) is
  M = max_c lse_c,  w_c = exp(lse_c - M),
  o = sum_c w_c * o_c / sum_c w_c,   lse = M + ln sum_c w_c
and equals the unsplit result.
"""
from __future__ import annotations

import numpy as np

from .attention import attend


def num_splits(seq_len: int, split_tokens: int) -> int:
    return -(-int(seq_len) // int(split_tokens)) if seq_len > 0 else 0


def split_partials(q, k, v, sm_scale: float, split_tokens: int):
    """(o [n, Hq, Dv], lse [n, Hq]) for each chunk of the request."""
    L = k.shape[0]
    parts_o, parts_l = [], []
    for c in range(num_splits(L, split_tokens)):
        sl = slice(c * split_tokens, min((c + 1) * split_tokens, L))
        o, lse = attend(q, k[sl], v[sl], sm_scale)
        parts_o.append(o)
        parts_l.append(lse)
    return np.stack(parts_o), np.stack(parts_l)


def combine(o_parts, lse_parts):
    """Merge chunk results: o_parts [n, Hq, Dv], lse_parts [n, Hq] -> (o, lse)."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    w = np.exp(lse_parts - M[None, :])
    den = w.sum(axis=0)
    o = (w[:, :, None] * o_parts).sum(axis=0) / den[:, None]
    return o, M + np.log(den)
