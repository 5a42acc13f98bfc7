"""GPU parity of the prefill -> decode page handoff (pkv_requantize_pages):
codes and tags must equal the oracle's bit for bit, unlisted pages and bad
pairs must be left alone, and a decode over handed-off pages must equal the
decode over the same tokens appended directly."""
import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import handoff, quant

pytestmark = pytest.mark.gpu
dev = "cuda"


def _bf16_pool(w, latent=False):
    """The workload's tokens in a BF16 cache, through pkv_append."""
    c = pkv.allocate_cache(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim_k, w.head_dim_v,
                           "bf16", latent, dev, poison=False)
    k = w.k_all(dev)
    v = None if latent else w.v_all(dev)
    pkv.pkv_append(c, k, v, torch.from_numpy(w.slots()).to(dev))
    return c


def _pool_values(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("latent", [False, True])
@pytest.mark.parametrize("per_head", [False, True])
def test_handoff_codes_scales_and_tags_bit_exact(latent, per_head):
    if latent:
        w = W.custom("ho_lat", 41, [200, 64, 130], hq=16, hkv=1, dk=576, dv=512, page=64,
                     latent=True)
    else:
        w = W.custom("ho", 42, [300, 77, 16, 161], hq=16, hkv=2, dk=128, dv=128, page=16,
                     per_head=per_head, outliers=True)
    src = _bf16_pool(w, latent)
    H, P = w.num_kv_heads, w.page_size
    n_dst = w.num_pages + 5
    dst = pkv.allocate_cache(n_dst, H, P, w.head_dim_k, w.head_dim_v, "fp8", latent, dev)
    rng = np.random.default_rng(5)
    dst.k_pool.copy_(torch.from_numpy(rng.integers(0, 256, size=tuple(dst.k_pool.shape),
                                                   dtype=np.uint8)).to(dev))
    if not latent:
        dst.v_pool.copy_(torch.from_numpy(rng.integers(0, 256, size=tuple(dst.v_pool.shape),
                                                       dtype=np.uint8)).to(dev))
    tags0 = rng.integers(0, 2**32, size=n_dst, dtype=np.uint64).astype(np.uint32)
    dst.page_tags = torch.from_numpy(tags0.view(np.int32).copy()).to(dev)
    # scales over the source pool viewed as [pages][heads][P * D]
    kview = src.k_pool.view(w.num_pages, H, P * w.head_dim_k)
    pkv.pkv_scales_from_amax(kview, per_head, dst.k_scale)
    kvals = _pool_values(src.k_pool)
    if per_head:
        ks_ref = np.array([quant.scale_from_amax(np.abs(kvals[:, h]).max()) for h in range(H)])
    else:
        ks_ref = np.full(H, quant.scale_from_amax(np.abs(kvals).max()))
    assert np.array_equal(dst.k_scale.cpu().numpy().view(np.uint32),
                          ks_ref.astype(np.float32).view(np.uint32))
    if latent:
        dst.v_scale = dst.k_scale
    else:
        vview = src.v_pool.view(w.num_pages, H, P * w.head_dim_v)
        # a smaller scale than amax / 448 for V, so some values saturate
        pkv.pkv_scales_from_amax(vview, per_head, dst.v_scale)
        dst.v_scale.mul_(0.5)
    # every source page to a shuffled destination page, plus bad pairs
    sp = list(range(w.num_pages)) + [-1, w.num_pages, 0]
    dp = list(rng.permutation(n_dst)[:w.num_pages]) + [0, 1, n_dst]
    new = rng.integers(0, 2**32, size=len(sp), dtype=np.uint64).astype(np.uint32)
    k0 = dst.k_pool.cpu().numpy()
    v0 = None if latent else dst.v_pool.cpu().numpy()
    pkv.pkv_requantize_pages(src, dst, torch.tensor(sp, dtype=torch.int32, device=dev),
                             torch.tensor(dp, dtype=torch.int32, device=dev),
                             torch.from_numpy(new.view(np.int32).copy()).to(dev))
    torch.cuda.synchronize()
    kc, tg = handoff.requantize_pages(kvals, k0, tags0, sp, dp, dst.k_scale.cpu().numpy(), new)
    assert np.array_equal(dst.k_pool.cpu().numpy(), kc)
    assert np.array_equal(dst.page_tags.cpu().numpy().view(np.uint32), tg)
    if not latent:
        vvals = _pool_values(src.v_pool)
        vs = dst.v_scale.cpu().numpy()
        vc, _ = handoff.requantize_pages(vvals, v0, None, sp, dp, vs)
        assert np.array_equal(dst.v_pool.cpu().numpy(), vc)
        assert np.any(np.abs(vvals) / vs[None, :, None, None] >= 448.0), \
            "the halved V scale should saturate some values"


def test_decode_over_handed_off_pages_equals_direct_append():
    w = W.custom("ho_dec", 43, [500, 260, 33], hq=64, hkv=8, dk=128, dv=128, page=16, split=128)
    src = _bf16_pool(w)
    # unwritten rows are zero on both sides (the BF16 pool is not poisoned)
    direct = pkv.allocate_cache(w.num_pages, w.num_kv_heads, w.page_size, 128, 128, "fp8", False,
                                dev, poison=False)
    k, v = w.k_all(dev), w.v_all(dev)
    pkv.pkv_scales_from_amax(k, False, direct.k_scale)
    pkv.pkv_scales_from_amax(v, False, direct.v_scale)
    pkv.pkv_append(direct, k, v, torch.from_numpy(w.slots()).to(dev))
    moved = pkv.allocate_cache(w.num_pages, w.num_kv_heads, w.page_size, 128, 128, "fp8", False, dev)
    moved.k_scale.copy_(direct.k_scale)
    moved.v_scale.copy_(direct.v_scale)
    pages = torch.arange(w.num_pages, dtype=torch.int32, device=dev)
    pkv.pkv_requantize_pages(src, moved, pages, pages)
    torch.cuda.synchronize()
    assert torch.equal(moved.k_pool, direct.k_pool) and torch.equal(moved.v_pool, direct.v_pool)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    q = w.q_values(dev)
    outs = []
    for c in (direct, moved):
        ds = pkv.DecodeStep(c, w.num_q_heads, w.batch, int(w.seq_lens.max()), 128, False, dev)
        outs.append(ds.attend(q, bt, lens, w.sm_scale, None).clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_handoff_rejects_bad_arguments():
    w = W.custom("ho_bad", 44, [40], hq=2, hkv=1, dk=64, dv=64, page=16)
    src = _bf16_pool(w)
    dst = pkv.allocate_cache(w.num_pages, 1, 16, 64, 64, "fp8", False, dev)
    pages = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_requantize_pages(dst, dst, pages, pages)      # source must be BF16
    other = pkv.allocate_cache(w.num_pages, 1, 32, 64, 64, "fp8", False, dev)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_requantize_pages(src, other, pages, pages)    # page sizes differ


def _special_bf16_pool(rng, pages, heads, page, dim, scales):
    """bf16 bit patterns [pages, heads, page, dim]: random values, then per
    16-value chunk a set of special values (NaN of both signs, quiet and
    signalling; infinities; signed zeros; the largest bf16; subnormals;
    exact e4m3 ties and the saturation edge under each head's scale)."""
    vals = rng.standard_normal((pages, heads, page, dim)).astype(np.float32) * 3.0
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    specials_common = [0x7F80, 0xFF80, 0x0000, 0x8000, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x007F]
    nans = [0x7FC0, 0xFFC0, 0x7F81, 0xFF81]

    def bf16_bits(x):
        return int((np.array([x], dtype=np.float32).view(np.uint32)[0] >> 16) & 0xFFFF)

    for h in range(heads):
        s = float(scales[h])
        # e4m3 midpoints (between 1 and 1.125, 2 and 2.25, the two smallest
        # subnormals) and the saturation edge, times s: exact when s is a power of two
        edge = [1.0625 * s, -1.0625 * s, 2.125 * s, 0.5 * 2.0 ** -9 * s, 1.5 * 2.0 ** -9 * s,
                448.0 * s, -448.0 * s, 464.0 * s, 447.0 * s, 480.0 * s]
        extra = [bf16_bits(e) for e in edge]
        flat = bits[:, h].reshape(-1)
        chunks = flat.size // 16
        for c in range(chunks):
            base = 16 * c
            if c % 3 == 0:     # a chunk holding a NaN
                flat[base + c % 16] = nans[c % len(nans)]
            pool = specials_common + extra
            for j in range(4):
                flat[base + (3 * j + c) % 16] = pool[(c * 4 + j) % len(pool)]
        bits[:, h] = flat.reshape(bits[:, h].shape)
    return bits


@pytest.mark.parametrize("scales", [(0.125, 2.0 ** -70), (0.0371, 2.0 ** 61), (2.0 ** -60, 2.0 ** 60)])
def test_handoff_special_values_bit_exact(scales):
    """NaN, infinities, signed zeros, bf16 extremes and subnormals, e4m3 ties
    and the saturation edge, under scales inside and outside [2^-60, 2^60]:
    every code equals the oracle's."""
    pages, H, P, D = 3, 2, 16, 128
    rng = np.random.default_rng(61)
    s32 = np.array(scales, dtype=np.float32)
    kb = _special_bf16_pool(rng, pages, H, P, D, s32)
    vb = _special_bf16_pool(rng, pages, H, P, D, s32[::-1].copy())
    src = pkv.allocate_cache(pages, H, P, D, D, "bf16", False, dev, poison=False)
    src.k_pool.copy_(torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16))
    src.v_pool.copy_(torch.from_numpy(vb.view(np.int16)).to(dev).view(torch.bfloat16))
    dst = pkv.allocate_cache(pages, H, P, D, D, "fp8", False, dev)
    dst.k_scale.copy_(torch.from_numpy(s32).to(dev))
    dst.v_scale.copy_(torch.from_numpy(s32[::-1].copy()).to(dev))
    pg = torch.arange(pages, dtype=torch.int32, device=dev)
    k0 = dst.k_pool.cpu().numpy()
    v0 = dst.v_pool.cpu().numpy()
    pkv.pkv_requantize_pages(src, dst, pg, pg)
    torch.cuda.synchronize()
    kv = (kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vv = (vb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kc, _ = handoff.requantize_pages(kv, k0, None, list(range(pages)), list(range(pages)), s32)
    vc, _ = handoff.requantize_pages(vv, v0, None, list(range(pages)), list(range(pages)),
                                     s32[::-1].copy())
    got_k, got_v = dst.k_pool.cpu().numpy(), dst.v_pool.cpu().numpy()
    bad = np.argwhere(got_k != kc)
    assert bad.size == 0, f"K codes differ at {bad[:4].tolist()}: {got_k[tuple(bad[0])]:#x} vs {kc[tuple(bad[0])]:#x}"
    bad = np.argwhere(got_v != vc)
    assert bad.size == 0, f"V codes differ at {bad[:4].tolist()}: {got_v[tuple(bad[0])]:#x} vs {vc[tuple(bad[0])]:#x}"


def test_handoff_every_bf16_value_bit_exact():
    """All 65536 bf16 bit patterns under six scales (one per kv head: powers
    of two, amax-style values and both ends of [2^-60, 2^60]): every code
    equals the oracle's."""
    H, P, D = 6, 16, 128
    pages = 65536 // (P * D)
    rng = np.random.default_rng(62)
    bits = np.empty((pages, H, P, D), dtype=np.uint16)
    for h in range(H):
        bits[:, h] = rng.permutation(65536).astype(np.uint16).reshape(pages, P, D)
    s32 = np.array([1.0, 0.125, 0.0371, 3.7 / 448.0, 2.0 ** -60, 2.0 ** 60], dtype=np.float32)
    src = pkv.allocate_cache(pages, H, P, D, D, "bf16", False, dev, poison=False)
    src.k_pool.copy_(torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16))
    src.v_pool.copy_(src.k_pool)
    dst = pkv.allocate_cache(pages, H, P, D, D, "fp8", False, dev)
    dst.k_scale.copy_(torch.from_numpy(s32).to(dev))
    dst.v_scale.copy_(torch.from_numpy(s32[::-1].copy()).to(dev))
    pg = torch.arange(pages, dtype=torch.int32, device=dev)
    pkv.pkv_requantize_pages(src, dst, pg, pg)
    torch.cuda.synchronize()
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for pool, sc in ((dst.k_pool, s32), (dst.v_pool, s32[::-1].copy())):
        got = pool.cpu().numpy()
        for h in range(H):
            want = quant.quantize(vals[:, h], sc[h])
            bad = np.argwhere(got[:, h] != want)
            assert bad.size == 0, (f"scale {sc[h]!r}: {len(bad)} codes differ, first x = "
                                   f"{vals[:, h][tuple(bad[0])]!r}")
