"""Buffers for one decode step and the four library calls that make it.

Allocation here is plain torch device memory (the library itself never
allocates); every computation is a libpkv launch on the current stream, in
the order the integrity rule needs ("Smaller, faster, safer", section
"Protecting a shared KV cache": the mapping is checked before decode reads):
    pkv_verify -> pkv_append -> pkv_decode_attn -> pkv_combine
with the first two as one launch (pkv_verify_append) when each request
appends one token; or, for one token per request at its last position, the
whole step in two launches (pkv_step_decode -> pkv_step_combine: the check
inside the decode, the append inside the merge).
"""
from __future__ import annotations

import torch

from ._binding import (Cache, pkv_append, pkv_combine, pkv_decode_attn, pkv_step_combine,
                       pkv_step_decode, pkv_suggest_split, pkv_verify, pkv_verify_append)

E4M3_NAN = 0x7F
BF16_NAN = 0x7FC0


def allocate_cache(num_pages: int, num_kv_heads: int, page_size: int, head_dim_k: int,
                   head_dim_v: int, kv_dtype: str = "fp8", latent: bool = False,
                   device="cuda", poison: bool = True, row_scales: bool = False) -> Cache:
    """Pools filled with NaN codes (so any read of an unwritten row shows),
    unit scales and zero tags. row_scales: also one scale per row, set at
    append (e4m3 with separate pools), poisoned with NaN like the codes."""
    shape_k = (num_pages, num_kv_heads, page_size, head_dim_k)
    shape_v = (num_pages, num_kv_heads, page_size, head_dim_v)
    if kv_dtype == "fp8":
        mk = lambda s: torch.full(s, E4M3_NAN if poison else 0, dtype=torch.uint8, device=device)
    elif kv_dtype == "bf16":
        mk = lambda s: torch.full(s, BF16_NAN if poison else 0, dtype=torch.int16,
                                  device=device).view(torch.bfloat16)
    else:
        raise ValueError(kv_dtype)
    k = mk(shape_k)
    v = None if latent else mk(shape_v)
    ones = lambda: torch.ones(num_kv_heads, dtype=torch.float32, device=device)
    rows = None
    if row_scales:
        if kv_dtype != "fp8" or latent:
            raise ValueError("row scales need an e4m3 cache with separate K and V pools")
        rows = [torch.full((num_pages, num_kv_heads, page_size), float("nan") if poison else 0.0,
                           dtype=torch.float32, device=device) for _ in range(2)]
    return Cache(k_pool=k, v_pool=v, k_scale=ones(), v_scale=ones(),
                 page_tags=torch.zeros(num_pages, dtype=torch.int32, device=device),
                 latent_dim_v=head_dim_v if latent else None,
                 k_row_scale=rows[0] if rows else None, v_row_scale=rows[1] if rows else None)


class DecodeStep:
    """Output and scratch buffers of a decode step for a fixed batch shape."""

    def __init__(self, cache: Cache, num_q_heads: int, batch: int, max_seq_len: int,
                 split_tokens: int | None = None, verify: bool = True, device="cuda",
                 total_tokens: int = 0):
        """total_tokens (the sum of the requests' lengths, 0 if unknown) only
        informs the split the library suggests when split_tokens is None."""
        self.cache = cache
        self.num_q_heads = num_q_heads
        self.batch = batch
        self.max_seq_len = max_seq_len
        self.split_tokens = split_tokens or pkv_suggest_split(
            cache, num_q_heads, batch, total_tokens, max_seq_len)
        self.max_splits = max(1, -(-max_seq_len // self.split_tokens))
        dv = cache.head_dim_v
        self.o_part = torch.empty((batch, num_q_heads, self.max_splits, dv), dtype=torch.float32,
                                  device=device)
        self.lse_part = torch.empty((batch, num_q_heads, self.max_splits), dtype=torch.float32,
                                    device=device)
        self.out = torch.empty((batch, num_q_heads, dv), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((batch, num_q_heads), dtype=torch.float32, device=device)
        self.verify = verify
        self.abort = torch.zeros(batch, dtype=torch.uint8, device=device)
        self.unit_flags = torch.zeros((batch, self.max_splits), dtype=torch.uint8, device=device)

    def run(self, q, block_table, expected_tags, seq_lens, sm_scale, k_new=None, v_new=None,
            slot=None, token_req=None):
        """One step. New tokens k_new[i] (v_new[i]) go to slot[i] for request
        token_req[i]; token_req None means one token per request, token b of
        request b, and then the check and the append are one launch."""
        c = self.cache
        abort = None
        if self.verify:
            if k_new is not None and token_req is None:
                pkv_verify_append(c, block_table, expected_tags, seq_lens, self.abort, k_new,
                                  v_new, slot)
                k_new = None
            else:
                pkv_verify(c, block_table, expected_tags, seq_lens, self.abort)
            abort = self.abort
        if k_new is not None:
            pkv_append(c, k_new, v_new, slot, token_req, abort)
        self.attend(q, block_table, seq_lens, sm_scale, abort)
        return self.out

    def attend(self, q, block_table, seq_lens, sm_scale, abort):
        pkv_decode_attn(self.cache, q, block_table, seq_lens, self.max_seq_len, abort, sm_scale,
                        self.split_tokens, self.o_part, self.lse_part)
        pkv_combine(self.o_part, self.lse_part, seq_lens, self.split_tokens, self.max_seq_len,
                    abort, self.out, self.lse)
        return self.out

    def step2(self, q, block_table, expected_tags, seq_lens, sm_scale, k_new, v_new=None):
        """One step in two launches: the tag check, the append of each
        request's new token (k_new[b], v_new[b]) at its last position
        (seq_lens[b] - 1), decode and merge; the same results as run() with
        those slots. Without verify (or with expected_tags None) there is no
        check and every request stands."""
        c = self.cache
        if not self.verify:
            expected_tags = None
        pkv_step_decode(c, q, k_new, v_new, block_table, expected_tags, seq_lens,
                        self.max_seq_len, sm_scale, self.split_tokens, self.o_part,
                        self.lse_part, self.unit_flags, self.abort)
        pkv_step_combine(c, k_new, v_new, block_table, expected_tags, seq_lens, self.max_seq_len,
                         self.split_tokens, self.o_part, self.lse_part, self.unit_flags,
                         self.abort, self.out, self.lse)
        return self.out
