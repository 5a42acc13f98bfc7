"""Seeded synthetic inputs of an INT4 weight-only linear layer in decode.

Holds no quantisation or matmul arithmetic: uniform random packed 4-bit
codes, positive bf16 group scales and bf16 activations, drawn by the
counter-based generator (hashgen) so that a GPU fill and a CPU sample of the
same rows hold the same bits.

Layout (the library's INT4 format): codes uint8 [n][k / 2], the code of
input k of row r in byte k / 2 of row r, even k in the low nibble; scales
bf16 [k / group][n] (group-major, so one group's scales of consecutive rows
are contiguous); activations bf16 [batch][k].
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import hashgen

S_CODES, S_SCALES, S_X = 1, 2, 3


@dataclass(frozen=True)
class Int4Layer:
    name: str
    seed: int
    n: int        # output features
    k: int        # input features
    batch: int    # decode tokens
    group: int = 128
    description: str = ""

    def codes(self, device="cpu", rows=None) -> torch.Tensor:
        """uint8 [n][k/2] (or [len(rows)][k/2] for a subset of rows)."""
        keys = hashgen.stream_keys(self.seed, S_CODES)
        half = self.k // 2
        if rows is None:
            return hashgen.u8_block(keys, self.n * half, device).view(self.n, half)
        r = torch.as_tensor(rows, dtype=torch.int64, device=device)
        idx = r[:, None] * half + torch.arange(half, dtype=torch.int64, device=device)[None, :]
        return hashgen.u8_from_index(keys, idx)

    def scales(self, device="cpu") -> torch.Tensor:
        """bf16 [k/group][n]: |N(0,1)| / 64, zeros replaced by 1/64 (all positive)."""
        keys = hashgen.stream_keys(self.seed, S_SCALES)
        v = hashgen.bf16_block(keys, (self.k // self.group) * self.n, device).abs()
        v = v * (1.0 / 64.0)  # a power of two: exact in bf16
        v = torch.where(v == 0, torch.full_like(v, 1.0 / 64.0), v)
        return v.view(self.k // self.group, self.n)

    def x(self, device="cpu") -> torch.Tensor:
        """bf16 [batch][k], N(0,1)."""
        keys = hashgen.stream_keys(self.seed, S_X)
        return hashgen.bf16_block(keys, self.batch * self.k, device).view(self.batch, self.k)


def int4_layer(batch: int, n: int = 8192, k: int = 8192, seed: int = 1007) -> Int4Layer:
    """A decode projection of hidden size 8192 (n x k INT4 weights, group 128)
    at `batch` concurrent tokens."""
    return Int4Layer(f"int4_{n}x{k}_b{batch}", seed, n, k, batch,
                     description=f"INT4 weights {n}x{k}, group 128, bf16 scales, B={batch}")


def int4_custom(name: str, seed: int, n: int, k: int, batch: int) -> Int4Layer:
    return Int4Layer(name, seed, n, k, batch, description=f"{n}x{k} B={batch}")
