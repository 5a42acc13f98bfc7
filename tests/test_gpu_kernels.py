"""GPU parity of the integer and byte steps: scales, quantise-on-append,
tag check. Every result must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import e4m3, quant, step, verify
from tests.gpu_state import State

pytestmark = pytest.mark.gpu
dev = "cuda"


def _f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- scales
@pytest.mark.parametrize("make", [W.tiny, lambda: W.gqa(2, 512), lambda: W.sweep(1),
                                  lambda: W.custom("ph", 7, [33, 200, 5], hq=8, hkv=4, dk=64, dv=64,
                                                   page=16, per_head=True, outliers=True)])
def test_scales_bit_exact(make):
    w = make()
    ks_ref, vs_ref = step.scales(w, "fp8")
    k = w.k_all(dev)
    ks = pkv.pkv_scales_from_amax(k, w.per_head_scales)
    assert np.array_equal(_f32_bits(ks.cpu().numpy()), _f32_bits(ks_ref))
    if not w.latent:
        vs = pkv.pkv_scales_from_amax(w.v_all(dev), w.per_head_scales)
        assert np.array_equal(_f32_bits(vs.cpu().numpy()), _f32_bits(vs_ref))


def test_scale_of_all_zero_tensor_is_one():
    x = torch.zeros((10, 2, 64), dtype=torch.bfloat16, device=dev)
    s = pkv.pkv_scales_from_amax(x, True)
    assert s.cpu().tolist() == [1.0, 1.0]


# ---------------------------------------------------------------- append
def _append_codes(values_bits: np.ndarray, s: float, dim: int = 128):
    """Append rows holding the given bf16 bit patterns through pkv_append and
    return the codes written, in input order."""
    n_rows = values_bits.size // dim
    P = 16
    n_pages = -(-n_rows // P)
    cache = pkv.allocate_cache(n_pages, 1, P, dim, dim, "fp8", device=dev)
    cache.k_scale.fill_(s)
    cache.v_scale.fill_(s)
    x = torch.from_numpy(values_bits.view(np.int16).reshape(n_rows, 1, dim).copy()).to(dev)
    x = x.view(torch.bfloat16)
    perm = np.random.default_rng(0).permutation(n_pages * P)[:n_rows].astype(np.int32)
    slot = torch.from_numpy(perm).to(dev)
    pkv.pkv_append(cache, x, x, slot)
    torch.cuda.synchronize()
    flat = cache.k_pool.view(n_pages * P, dim).cpu().numpy()
    vflat = cache.v_pool.view(n_pages * P, dim).cpu().numpy()
    assert np.array_equal(flat, vflat)
    return flat[perm].reshape(-1)


@pytest.mark.parametrize("s", [1.0, 4.90625 / 448, 96.0 / 448, 2.0**-7, 3.0, 1e-20, 1e20])
def test_append_every_bf16_pattern_bit_exact(s):
    s32 = np.float32(s)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = _append_codes(bits, float(s32))
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    ref = quant.quantize(x, s32)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(bits[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


def test_append_ties_bit_exact():
    """bf16 values landing exactly on e4m3 midpoints after division by 1."""
    mags = e4m3.DECODE[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    bits = (mids.view(np.uint32) >> 16).astype(np.uint16)
    exact = ((bits.astype(np.uint32) << 16).view(np.float32) == mids)
    bits = np.concatenate([bits[exact], bits[exact] | 0x8000])
    pad = (-bits.size) % 128
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)])
    got = _append_codes(bits, 1.0)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(got, quant.quantize(x, np.float32(1.0)))


@pytest.mark.parametrize("make", [W.tiny, lambda: W.custom("lat", 3, [70, 129, 1], hq=16, hkv=1, dk=576,
                                                            dv=512, page=64, latent=True)])
def test_bulk_fill_whole_pool_bit_exact(make):
    w = make()
    st = State(w, "fp8")
    torch.cuda.synchronize()
    ks, vs = step.scales(w, "fp8")
    exp_k = np.full(tuple(st.cache.k_pool.shape), 0x7F, dtype=np.uint8)
    exp_v = None if w.latent else np.full(tuple(st.cache.v_pool.shape), 0x7F, dtype=np.uint8)
    for b in range(w.batch):
        kc, vc = step.request_codes(w, b, ks, vs)
        t = np.arange(w.seq_lens[b])
        pages, rows = w.block_table[b, t // w.page_size], t % w.page_size
        exp_k[pages, :, rows, :] = kc
        if exp_v is not None:
            exp_v[pages, :, rows, :] = vc
    assert np.array_equal(st.cache.k_pool.cpu().numpy(), exp_k)
    if exp_v is not None:
        assert np.array_equal(st.cache.v_pool.cpu().numpy(), exp_v)


def test_append_skips_negative_slots_and_aborted_requests():
    cache = pkv.allocate_cache(4, 2, 16, 64, 64, "fp8", device=dev)
    x = torch.ones((4, 2, 64), dtype=torch.bfloat16, device=dev)
    slot = torch.tensor([0, -1, 17, 63], dtype=torch.int32, device=dev)
    req = torch.tensor([0, 0, 1, 2], dtype=torch.int32, device=dev)
    abort = torch.tensor([0, 1, 0], dtype=torch.uint8, device=dev)
    pkv.pkv_append(cache, x, x, slot, req, abort)
    torch.cuda.synchronize()
    flat = cache.k_pool.permute(0, 2, 1, 3).reshape(64, 2, 64).cpu().numpy()
    one = int(quant.quantize(np.float32(1.0), np.float32(1.0)))
    written = {0, 63}
    for s in range(64):
        assert np.all(flat[s] == (one if s in written else 0x7F)), s


def test_bf16_append_is_a_copy():
    w = W.custom("b", 4, [40, 3], hq=4, hkv=2, dk=128, dv=128, page=16)
    st = State(w, "bf16")
    for b in range(w.batch):
        k, v = st.request_pool(b)
        assert torch.equal(k.view(torch.int16).cpu(), w.k_values(b).view(torch.int16))
        assert torch.equal(v.view(torch.int16).cpu(), w.v_values(b).view(torch.int16))


# ---------------------------------------------------------------- verify
def _gpu_flags(w, bt=None, exp=None, tags=None):
    cache = pkv.allocate_cache(w.num_pages, 1, w.page_size, 16, 16, "fp8", device=dev)
    tags = w.page_tags if tags is None else tags
    cache.page_tags = torch.from_numpy(tags.view(np.int32).copy()).to(dev)
    bt = w.block_table if bt is None else bt
    exp = w.expected_tags if exp is None else exp
    out = torch.full((w.batch,), 7, dtype=torch.uint8, device=dev)
    pkv.pkv_verify(cache, torch.from_numpy(np.ascontiguousarray(bt, dtype=np.int32)).to(dev),
                   torch.from_numpy(np.ascontiguousarray(exp, dtype=np.uint32).view(np.int32)).to(dev),
                   torch.from_numpy(w.seq_lens).to(dev), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("make", [W.tiny, lambda: W.tiny(True), W.mla, lambda: W.sweep(64),
                                  W.long_context])
def test_verify_flags_bit_exact(make):
    w = make()
    ref = verify.verify(w.page_tags, w.block_table, w.expected_tags, w.seq_lens, w.page_size)
    assert np.array_equal(_gpu_flags(w), ref)


def test_verify_mla_aborts_exactly_the_readers_of_reallocated_pages():
    w = W.mla()
    got = _gpu_flags(w)
    readers = set()
    for b in range(w.batch):
        n = -(-int(w.seq_lens[b]) // w.page_size)
        if np.isin(w.block_table[b, :n], w.reallocated_pages).any():
            readers.add(b)
    assert set(np.nonzero(got)[0].tolist()) == readers and len(readers) >= 1


def test_verify_random_corruptions():
    rng = np.random.default_rng(21)
    for trial in range(20):
        lens = rng.integers(0, 300, size=int(rng.integers(1, 70)))
        w = W.custom(f"r{trial}", 2000 + trial, np.maximum(lens, 1), hq=1, hkv=1, dk=16, dv=16,
                     page=16, pool_pages=int(np.sum(-(-np.maximum(lens, 1) // 16))) + 5)
        w.seq_lens[:] = lens  # empty requests allowed here
        bt = w.block_table.copy()
        exp = w.expected_tags.copy()
        tags = w.page_tags.copy()
        k = int(rng.integers(0, 4))
        for _ in range(k):
            b, j = int(rng.integers(0, w.batch)), int(rng.integers(0, bt.shape[1]))
            kind = rng.integers(0, 4)
            if kind == 0:
                bt[b, j] = w.num_pages + int(rng.integers(0, 5))
            elif kind == 1:
                bt[b, j] = -1
            elif kind == 2:
                exp[b, j] ^= 1
            else:
                tags[int(rng.integers(0, w.num_pages))] += 1
        ref = verify.verify(tags, bt, exp, w.seq_lens, w.page_size)
        assert np.array_equal(_gpu_flags(w, bt, exp, tags), ref), trial


def test_verify_long_rows_across_rounds():
    """Rows of 5000 entries (more than two 2048-entry rounds of the kernel),
    corruptions exactly at round edges, and a request longer than its row."""
    P = 16
    n_ent = 5000
    B = 9
    rng = np.random.default_rng(5)
    num_pages = B * n_ent + 7
    perm = rng.permutation(num_pages)[:B * n_ent].reshape(B, n_ent).astype(np.int32)
    tags = rng.integers(0, 2**32, size=num_pages, dtype=np.uint64).astype(np.uint32)
    exp = tags[perm].copy()
    lens = np.full(B, n_ent * P, dtype=np.int32)
    edges = [0, 2047, 2048, 4095, 4096, 4999]
    for b, j in enumerate(edges):
        exp[b, j] ^= 0x80000000
    lens[6] = n_ent * P - 3           # clean, ragged last page
    lens[7] = n_ent * P + 1           # needs one entry more than the row holds
    bt = perm.copy()
    bt[8, 4999] = num_pages           # out-of-pool id in the last entry
    w = W.custom("vlong", 4242, [16] * B, hq=1, hkv=1, dk=16, dv=16, page=P, pool_pages=num_pages)
    w.seq_lens[:] = lens
    ref = verify.verify(tags, bt, exp, lens, P)
    assert ref.tolist() == [1] * 6 + [0, 1, 1]
    assert np.array_equal(_gpu_flags(w, bt, exp, tags), ref)


# ------------------------------------------------- check and append in one launch
def _pools(c):
    out = [c.k_pool.view(torch.uint8).clone()]
    if c.v_pool is not None:
        out.append(c.v_pool.view(torch.uint8).clone())
    if c.k_row_scale is not None:
        out += [c.k_row_scale.clone(), c.v_row_scale.clone()]
    return out


@pytest.mark.parametrize("kv,rows,latent", [("fp8", False, False), ("bf16", False, False),
                                             ("fp8", True, False), ("fp8", False, True),
                                             ("bf16", False, True)])
def test_verify_append_equals_verify_then_append(kv, rows, latent):
    """pkv_verify_append gives the flags of pkv_verify and the pools of
    pkv_append with each request's token and the flags, byte for byte:
    aborted requests (reallocated pages) write nothing, a negative slot
    writes nothing."""
    dk, dv = (576, 512) if latent else (128, 128)
    w = W.custom(f"va_{kv}_{rows}_{latent}", 95, [300, 17, 1000, 64, 2048, 5], hq=128 if latent else 16,
                 hkv=1 if latent else 2, dk=dk, dv=dv, page=64 if latent else 16, latent=latent,
                 n_realloc=2, sm_scale=1 / 24 if latent else None)
    flags = step.flags(w)
    assert flags.any() and not flags.all()
    a = State(w, kv, row_scales=rows)
    b = State(w, kv, row_scales=rows)
    slot = a.new_slot.clone()
    slot[3] = -1
    # new rows that differ from what the bulk fill wrote there
    k_new = torch.flip(a.new_k, dims=[0]).contiguous()
    v_new = None if latent else torch.flip(a.new_v, dims=[0]).contiguous()
    ab_a = torch.full((w.batch,), 7, dtype=torch.uint8, device=dev)
    ab_b = torch.full((w.batch,), 7, dtype=torch.uint8, device=dev)
    pkv.pkv_verify_append(a.cache, a.block_table, a.expected, a.seq_lens, ab_a, k_new, v_new, slot)
    pkv.pkv_verify(b.cache, b.block_table, b.expected, b.seq_lens, ab_b)
    pkv.pkv_append(b.cache, k_new, v_new, slot, b.new_req, ab_b)
    torch.cuda.synchronize()
    assert np.array_equal(ab_a.cpu().numpy(), flags) and torch.equal(ab_a, ab_b)
    for x, y in zip(_pools(a.cache), _pools(b.cache)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    # and the step through the fused call decodes as the separate calls do
    oa = a.run(fused=True).clone()
    ob = b.run(fused=False).clone()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
