"""Device state for a workload, built only through the library's entry points
(scales, bulk append), plus comparison helpers for the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_fp8_amd as pkv

ATOL, RTOL = 2e-3, 1e-2
# lse (natural log): the kernels that add bf16-rounded numerators to the
# denominator are off by up to 2^-9 in l, so up to about 2e-3 in ln l
LSE_ATOL = 4e-3


class State:
    def __init__(self, w, kv_dtype: str, split_tokens: int | None = None, verify: bool = True,
                 device="cuda", row_scales: bool = False):
        self.w = w
        self.kv_dtype = kv_dtype
        c = pkv.allocate_cache(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim_k,
                               w.head_dim_v, kv_dtype, w.latent, device, row_scales=row_scales)
        self.cache = c
        k = w.k_all(device)
        v = None if w.latent else w.v_all(device)
        if kv_dtype == "fp8" and not row_scales:
            pkv.pkv_scales_from_amax(k, w.per_head_scales, c.k_scale)
            if w.latent:
                c.v_scale = c.k_scale
            else:
                pkv.pkv_scales_from_amax(v, w.per_head_scales, c.v_scale)
        self.slot = torch.from_numpy(w.slots()).to(device)
        self.token_req = torch.from_numpy(w.token_request()).to(device)
        pkv.pkv_append(c, k, v, self.slot)  # bulk fill of every token
        self.k_all, self.v_all = k, v
        c.page_tags = torch.from_numpy(w.page_tags.view(np.int32).copy()).to(device)
        self.block_table = torch.from_numpy(w.block_table).to(device)
        self.expected = torch.from_numpy(w.expected_tags.view(np.int32).copy()).to(device)
        self.seq_lens = torch.from_numpy(w.seq_lens).to(device)
        self.q = w.q_values(device)
        self.max_seq_len = int(w.seq_lens.max())
        split = split_tokens or w.split_tokens
        self.step = pkv.DecodeStep(c, w.num_q_heads, w.batch, self.max_seq_len, split, verify,
                                   device, total_tokens=int(w.seq_lens.sum()))
        # the token appended this step: each request's last token
        off = w.token_offsets()
        last = torch.from_numpy(off[1:] - 1).to(device)
        self.new_k = k[last].contiguous()
        self.new_v = None if v is None else v[last].contiguous()
        self.new_slot = self.slot[last].contiguous()
        self.new_req = torch.arange(w.batch, dtype=torch.int32, device=device)

    def run(self, fused: bool = True):
        """The step; fused: the check and the append in one launch
        (pkv_verify_append), else the two separate calls."""
        out = self.step.run(self.q, self.block_table, self.expected, self.seq_lens,
                            self.w.sm_scale, self.new_k, self.new_v, self.new_slot,
                            None if fused else self.new_req)
        torch.cuda.synchronize()
        return out

    def request_pool(self, b: int):
        """The cache rows request b reads, gathered on the device: [L, Hkv, D]."""
        w = self.w
        L = int(w.seq_lens[b])
        t = torch.arange(L, device=self.q.device)
        pages = self.block_table[b].long()[t // w.page_size]
        rows = t % w.page_size
        k = self.cache.k_pool[pages, :, rows, :]
        v = None if w.latent else self.cache.v_pool[pages, :, rows, :]
        return k, v


def assert_close(gpu, ref, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    tol = ATOL + RTOL * np.abs(r)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} outside tolerance; "
                             f"first at {i.tolist()}: gpu={g[bad][:5]} ref={r[bad][:5]}; "
                             f"max err {err.max():.3e}")


def assert_lse_close(gpu, ref, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(g) & np.isneginf(r)
    err = np.where(both_inf, 0.0, np.abs(g - r))
    bad = ~(err <= LSE_ATOL)
    if bad.any():
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} lse outside {LSE_ATOL}; "
                             f"gpu={g[bad][:5]} ref={r[bad][:5]}; max err {np.nanmax(err):.3e}")
