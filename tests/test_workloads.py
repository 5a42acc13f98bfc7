"""The seeded input generators: determinism, structure, and the exact amax
shortcut against a full scan."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads import hashgen


def test_hash_inverse_and_torch_numpy_agree():
    rng = np.random.default_rng(0)
    x = rng.integers(0, 2**32, size=100_000, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(hashgen.unmix32_np(hashgen.mix32_np(x)), x)
    t = hashgen.mix32_t(torch.from_numpy(x.astype(np.int64)))
    assert np.array_equal(t.numpy(), hashgen.mix32_np(x).astype(np.int64))


def test_table_symmetric_monotone_and_normal():
    tab = hashgen.normal_table()
    v = torch.from_numpy(tab.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.all(np.diff(v) >= 0)
    assert np.array_equal(v, -v[::-1])
    assert abs(v.mean()) < 1e-6 and abs(v.std() - 1) < 2e-3


def test_values_deterministic_and_roughly_standard_normal():
    keys = hashgen.stream_keys(123, 2, 0)
    a = hashgen.bf16_block(keys, 1 << 18)
    b = hashgen.bf16_block(keys, 1 << 18)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    x = a.double()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_outlier_fraction_and_magnitude():
    keys = hashgen.stream_keys(7, 2, 0)
    n = 1 << 21
    x = hashgen.bf16_block(keys, n, outliers=True).double()
    y = hashgen.bf16_block(keys, n, outliers=False).double()
    frac = (x != y).double().mean().item()
    assert 0.0007 < frac < 0.0013
    r = (x[x != y] / y[x != y])
    assert torch.all((r - 20).abs() < 0.2)


@pytest.mark.parametrize("outliers", [False, True])
def test_amax_shortcut_equals_scan(outliers):
    keys = hashgen.stream_keys(99, 2, 3)
    for n, sel in [(3 << 20, None), (5 << 20, lambda i: (i // 128) % 8 == 5)]:
        fast = hashgen.amax_bits(keys, n, sel, outliers, brute_limit=0)
        slow = hashgen.amax_bits(keys, n, sel, outliers, brute_limit=1 << 30)
        assert fast == slow


def test_tiny_layout():
    w = W.tiny()
    assert w.seq_lens.tolist() == [37, 64]
    used = w.block_table[w.block_table >= 0]
    assert sorted(used.tolist()) == sorted(set(used.tolist()))  # no page twice
    assert used.size == 7 and w.num_pages == 16
    assert w.reallocated_pages.size == 1 and w.reallocated_pages[0] in used


def test_sweep_layout():
    for B in (1, 8):
        w = W.sweep(B)
        assert w.batch == B and np.all((w.seq_lens >= 2048) & (w.seq_lens <= 32768))
        used = w.block_table[w.block_table >= 0]
        assert np.array_equal(np.sort(used), np.arange(w.num_pages))  # exact pool
        assert w.reallocated_pages.size == 0 and w.per_head_scales


def test_mla_layout_and_corruption():
    w = W.mla()
    assert w.batch == 64 and w.latent and w.head_dim_k == 576 and w.head_dim_v == 512
    assert np.all((w.seq_lens >= 1) & (w.seq_lens <= 65536))
    assert 3000 < np.median(w.seq_lens) < 20000
    used = W.in_use_pages(w.block_table, w.seq_lens, w.page_size)
    assert w.reallocated_pages.size == max(1, round(0.001 * used.size))
    assert np.all(np.isin(w.reallocated_pages, used))


def test_slots_and_values_agree_between_whole_and_sampled_generation():
    w = W.custom("t", 5, [5, 17, 33], hq=4, hkv=2, dk=16, dv=16, page=16)
    ka = w.k_all()
    off = w.token_offsets()
    for b in range(w.batch):
        assert torch.equal(ka[off[b]:off[b + 1]].view(torch.int16), w.k_values(b).view(torch.int16))
    kh = w.k_values(1, heads=[1], tokens=[3, 9])
    assert torch.equal(kh[:, 0].view(torch.int16), ka[off[1] + np.array([3, 9]), 1].view(torch.int16))
    s = w.slots()
    P = 16
    for b in range(w.batch):
        for t in range(w.seq_lens[b]):
            assert s[off[b] + t] == w.block_table[b, t // P] * P + t % P
