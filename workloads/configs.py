"""Seeded synthetic decode workloads (inputs only; no method arithmetic).

Each workload is a batch of decode requests over a paged KV pool:
  * context lengths ``seq_lens`` (they count the token appended this step),
  * a block table mapping each request's logical pages to physical pool pages,
  * per-page pool tags and the tags each request recorded when its pages
    were handed out, with a chosen set of pool pages "reallocated" (their
    tag bumped by one, modulo 2**32) to exercise the integrity check,
  * bf16 K, V and Q values from ``workloads.hashgen`` (per-request streams,
    so any request or head can be regenerated alone, on CPU or GPU).

The workloads stand in for the decode measurements of "Smaller, faster,
safer: running Kimi and GLM at scale" (table in "Quantizing the KV cache":
concurrency 1 to 64; table in "Protecting a shared KV cache": 8,192-token
inputs, 1,000-token outputs). Shapes follow the five benchmark
configurations of this library; the lognormal spread, corruption count and
outlier rule are stated readings of those configurations.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import hashgen

# stream ids (fixed draw order: lengths, pages, K, V, Q, tags, corruption)
S_LEN, S_PERM, S_K, S_V, S_Q, S_TAGS, S_CORRUPT = range(7)


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    latent: bool  # one latent row per token; V is its first head_dim_v values
    page_size: int
    num_pages: int
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_pages], -1 beyond a request's pages
    page_tags: np.ndarray  # uint32 [num_pages], pool side after reallocations
    expected_tags: np.ndarray  # uint32 [B, max_pages], recorded by the server
    reallocated_pages: np.ndarray  # int64, pool pages whose tag was bumped
    sm_scale: float
    split_tokens: int | None
    per_head_scales: bool
    outliers: bool
    description: str = ""
    _amax_cache: dict = field(default_factory=dict, repr=False)

    # ---------------------------------------------------------------- shape
    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def token_offsets(self) -> np.ndarray:
        off = np.zeros(self.batch + 1, dtype=np.int64)
        off[1:] = np.cumsum(self.seq_lens.astype(np.int64))
        return off

    def slots(self) -> np.ndarray:
        """int32 pool slot (page * P + row) of every token, request-major."""
        P = self.page_size
        out = np.empty(self.total_tokens, dtype=np.int32)
        off = self.token_offsets()
        for b in range(self.batch):
            t = np.arange(self.seq_lens[b], dtype=np.int64)
            out[off[b]:off[b + 1]] = self.block_table[b, t // P] * P + t % P
        return out

    def token_request(self) -> np.ndarray:
        return np.repeat(np.arange(self.batch, dtype=np.int32), self.seq_lens.astype(np.int64))

    # --------------------------------------------------------------- values
    def _keys(self, stream: int, b: int = 0):
        return hashgen.stream_keys(self.seed, stream, b)

    def _row_values(self, stream: int, b: int, width: int, heads, tokens, device):
        """bf16 [len(tokens), len(heads), width] for request b's K or V stream."""
        H = self.num_kv_heads
        L = int(self.seq_lens[b])
        t = torch.arange(L, dtype=torch.int64, device=device) if tokens is None else \
            torch.as_tensor(np.asarray(tokens, dtype=np.int64), device=device)
        h = torch.arange(H, dtype=torch.int64, device=device) if heads is None else \
            torch.as_tensor(np.asarray(heads, dtype=np.int64), device=device)
        d = torch.arange(width, dtype=torch.int64, device=device)
        idx = (t[:, None, None] * H + h[None, :, None]) * width + d[None, None, :]
        return hashgen.bf16_from_index(self._keys(stream, b), idx, self.outliers)

    def k_values(self, b: int, heads=None, tokens=None, device="cpu") -> torch.Tensor:
        return self._row_values(S_K, b, self.head_dim_k, heads, tokens, device)

    def v_values(self, b: int, heads=None, tokens=None, device="cpu") -> torch.Tensor:
        if self.latent:
            raise ValueError("latent workloads have no separate V stream")
        return self._row_values(S_V, b, self.head_dim_v, heads, tokens, device)

    def _all_rows(self, stream: int, width: int, device) -> torch.Tensor:
        H = self.num_kv_heads
        out = torch.empty((self.total_tokens, H, width), dtype=torch.bfloat16, device=device)
        off = self.token_offsets()
        for b in range(self.batch):
            n = int(self.seq_lens[b]) * H * width
            out[off[b]:off[b + 1]] = hashgen.bf16_block(
                self._keys(stream, b), n, device, self.outliers).view(-1, H, width)
        return out

    def k_all(self, device="cpu") -> torch.Tensor:
        """bf16 [total_tokens, Hkv, Dk], request-major (matches ``slots``)."""
        return self._all_rows(S_K, self.head_dim_k, device)

    def v_all(self, device="cpu") -> torch.Tensor:
        if self.latent:
            raise ValueError("latent workloads have no separate V stream")
        return self._all_rows(S_V, self.head_dim_v, device)

    def q_values(self, device="cpu") -> torch.Tensor:
        """bf16 [B, Hq, Dk]; queries never carry outliers."""
        n = self.batch * self.num_q_heads * self.head_dim_k
        return hashgen.bf16_block(self._keys(S_Q), n, device).view(
            self.batch, self.num_q_heads, self.head_dim_k)

    # The same values as raw bf16 bit patterns in NumPy uint16 arrays (for
    # consumers that take no torch tensors).
    def k_bits(self, b: int, heads=None, tokens=None) -> np.ndarray:
        return _bits(self.k_values(b, heads=heads, tokens=tokens))

    def v_bits(self, b: int, heads=None, tokens=None) -> np.ndarray:
        return _bits(self.v_values(b, heads=heads, tokens=tokens))

    def q_bits(self) -> np.ndarray:
        return _bits(self.q_values())

    # ---------------------------------------------------------------- amax
    def amax(self, which: str, head: int | None = None) -> float:
        """Exact max |x| over every K (or V) value of every request, or of one
        kv head. A statistic of the inputs, found without a full scan."""
        key = (which, head)
        if key not in self._amax_cache:
            stream = {"k": S_K, "v": S_V}[which]
            width = self.head_dim_k if which == "k" else self.head_dim_v
            H = self.num_kv_heads
            sel = None
            if head is not None:
                sel = (lambda i, h=head: (i // width) % H == h)
            best = 0
            for b in range(self.batch):
                n = int(self.seq_lens[b]) * H * width
                best = max(best, hashgen.amax_bits(self._keys(stream, b), n, sel, self.outliers))
            self._amax_cache[key] = float(
                np.array([best << 16], dtype=np.uint32).view(np.float32)[0])
        return self._amax_cache[key]


# ----------------------------------------------------------------------------
# construction helpers
# ----------------------------------------------------------------------------
def _bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU bf16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream, 7919])


def _layout(seed, seq_lens, page_size, pool_pages=None, perm=None):
    B = len(seq_lens)
    need = [-(-int(L) // page_size) for L in seq_lens]
    total = sum(need)
    num_pages = total if pool_pages is None else pool_pages
    if num_pages < total:
        raise ValueError("pool too small")
    if perm is None:
        perm = _rng(seed, S_PERM).permutation(num_pages)
    max_pages = max(need)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[o:o + n]
        o += n
    tags = _rng(seed, S_TAGS).integers(0, 2**32, size=num_pages, dtype=np.uint64).astype(np.uint32)
    exp = np.zeros((B, max_pages), dtype=np.uint32)
    for b, n in enumerate(need):
        exp[b, :n] = tags[bt[b, :n]]
    return num_pages, bt, tags, exp


def _reallocate(tags: np.ndarray, pages: np.ndarray) -> np.ndarray:
    """Pool-side tag bump of the given pages (a reallocation)."""
    out = tags.copy()
    for p in pages:
        out[p] = np.uint32((int(out[p]) + 1) & 0xFFFFFFFF)
    return out


def _make(name, seed, seq_lens, *, hq, hkv, dk, dv, latent, page, pool_pages=None,
          perm=None, sm_scale, split=None, per_head=False, outliers=False,
          realloc=None, description=""):
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    num_pages, bt, tags, exp = _layout(seed, seq_lens, page, pool_pages, perm)
    pages = np.zeros(0, dtype=np.int64) if realloc is None else np.asarray(realloc(bt, seq_lens, page), dtype=np.int64)
    pool_tags = _reallocate(tags, pages)
    return Workload(name=name, seed=seed, batch=len(seq_lens), num_q_heads=hq,
                    num_kv_heads=hkv, head_dim_k=dk, head_dim_v=dv, latent=latent,
                    page_size=page, num_pages=num_pages, seq_lens=seq_lens,
                    block_table=bt, page_tags=pool_tags, expected_tags=exp,
                    reallocated_pages=pages, sm_scale=float(sm_scale),
                    split_tokens=split, per_head_scales=per_head, outliers=outliers,
                    description=description)


def in_use_pages(bt: np.ndarray, seq_lens: np.ndarray, page: int) -> np.ndarray:
    out = [bt[b, :-(-int(L) // page)] for b, L in enumerate(seq_lens)]
    return np.unique(np.concatenate(out)) if out else np.zeros(0, dtype=np.int64)


# ----------------------------------------------------------------------------
# the configurations
# ----------------------------------------------------------------------------
def tiny(bump_unused: bool = False) -> Workload:
    """2 requests (37 and 64 tokens), 4 q heads / 1 kv head, head dim 64,
    page 16, a 16-page pool in seeded random permutation; one in-use page is
    reallocated (or, with ``bump_unused``, one page no request reads)."""
    seed = 1000
    perm = _rng(seed, S_PERM).permutation(16)

    def pick(bt, lens, P):
        used = in_use_pages(bt, lens, P)
        pool = used if not bump_unused else np.setdiff1d(np.arange(16), used)
        return [int(_rng(seed, S_CORRUPT).choice(pool))]

    return _make("tiny" + ("_unused_bump" if bump_unused else ""), seed, [37, 64],
                 hq=4, hkv=1, dk=64, dv=64, latent=False, page=16, pool_pages=16, perm=perm,
                 sm_scale=1 / math.sqrt(64), realloc=pick,
                 description="B=2 L=(37,64) Hq=4 Hkv=1 D=64 P=16 pool=16")


def gqa(batch: int = 8, ctx: int = 4096) -> Workload:
    """batch 8, context 4096, 64 q / 8 kv heads, head dim 128, page 16."""
    return _make(f"gqa_b{batch}", 1001, [ctx] * batch, hq=64, hkv=8, dk=128, dv=128,
                 latent=False, page=16, sm_scale=1 / math.sqrt(128),
                 description=f"B={batch} L={ctx} Hq=64 Hkv=8 D=128 P=16")


SWEEP_BATCHES = (1, 8, 16, 32, 64)


def sweep(batch: int) -> Workload:
    """Concurrency sweep point: contexts uniform on [2048, 32768], 64 q / 8 kv
    heads, head dim 128, page 16, pool sized exactly for the requests, pages
    scattered, per-(K|V, kv head) scales, tag check on."""
    seed = 1002 + batch
    lens = _rng(seed, S_LEN).integers(2048, 32768 + 1, size=batch)
    return _make(f"sweep_b{batch}", seed, lens, hq=64, hkv=8, dk=128, dv=128, latent=False,
                 page=16, sm_scale=1 / math.sqrt(128), per_head=True,
                 description=f"B={batch} L~U[2048,32768] Hq=64 Hkv=8 D=128 P=16 per-head scales")


def long_context(batch: int = 4, ctx: int = 131072) -> Workload:
    """batch 4, context 131072, 64 q / 8 kv heads, head dim 128, page 64,
    0.1% of K and V elements scaled by 20 before rounding, 256-token splits."""
    return _make(f"long_b{batch}", 1003, [ctx] * batch, hq=64, hkv=8, dk=128, dv=128,
                 latent=False, page=64, sm_scale=1 / math.sqrt(128), split=256,
                 outliers=True,
                 description=f"B={batch} L={ctx} Hq=64 Hkv=8 D=128 P=64 split=256 outliers")


def mla(batch: int = 64) -> Workload:
    """batch 64, 128 q heads over one latent kv head of width 576 (V = first
    512), contexts lognormal (median 8192, sigma 1, capped at 65536), page 64;
    0.1% of in-use pages (at least one) reallocated."""
    seed = 1004
    z = _rng(seed, S_LEN).standard_normal(batch)
    lens = np.minimum(65536, np.maximum(1, np.rint(8192 * np.exp(z)))).astype(np.int64)

    def pick(bt, lens_, P):
        used = in_use_pages(bt, lens_, P)
        n = max(1, int(round(0.001 * used.size)))
        return np.sort(_rng(seed, S_CORRUPT).choice(used, size=n, replace=False))

    return _make(f"mla_b{batch}", seed, lens, hq=128, hkv=1, dk=576, dv=512, latent=True,
                 page=64, sm_scale=1 / math.sqrt(576), realloc=pick,
                 description=f"B={batch} L~lognormal(8192) cap 65536 Hq=128 latent 576/512 P=64")


def integrity_cost(batch: int) -> Workload:
    """Stand-in for the integrity-cost table: 8,192-token prompts half-way
    through a 1,000-token answer (L = 8692), GQA shape, page 16."""
    return _make(f"integrity_b{batch}", 1006, [8692] * batch, hq=64, hkv=8, dk=128, dv=128,
                 latent=False, page=16, sm_scale=1 / math.sqrt(128),
                 description=f"B={batch} L=8692 Hq=64 Hkv=8 D=128 P=16")


def custom(name, seed, seq_lens, *, hq, hkv, dk, dv, page, latent=False, pool_pages=None,
           sm_scale=None, split=None, per_head=False, outliers=False, n_realloc=0) -> Workload:
    """Small ad-hoc workloads for property and edge-case tests."""
    def pick(bt, lens, P):
        used = in_use_pages(bt, lens, P)
        if n_realloc <= 0 or used.size == 0:
            return []
        return np.sort(_rng(seed, S_CORRUPT).choice(used, size=min(n_realloc, used.size), replace=False))

    return _make(name, seed, seq_lens, hq=hq, hkv=hkv, dk=dk, dv=dv, latent=latent, page=page,
                 pool_pages=pool_pages, sm_scale=(1 / math.sqrt(dk)) if sm_scale is None else sm_scale,
                 split=split, per_head=per_head, outliers=outliers, realloc=pick)
