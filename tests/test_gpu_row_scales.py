"""GPU parity of scales set at append, one per cached row: the codes and row
scales pkv_append writes, bit for bit against the oracle's row quantiser
(oracle.quant.quantize_rows), and decode over such a cache against float64
attention over the rows dequantised with their own scales, within
|gpu - ref| <= 2e-3 + 1e-2 |ref|."""
import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import attention, quant, step
from tests.gpu_state import State, assert_close

pytestmark = pytest.mark.gpu
dev = "cuda"


def _pool_rows(st, b):
    """The codes and row scales request b's tokens occupy in the pools."""
    w = st.w
    off = w.token_offsets()
    slots = torch.from_numpy(w.slots()[off[b]:off[b + 1]].astype(np.int64)).to(dev)
    page, row = slots // w.page_size, slots % w.page_size
    c = st.cache
    kc = c.k_pool[page, :, row, :].cpu().numpy()          # [L, H, D]
    vc = c.v_pool[page, :, row, :].cpu().numpy()
    ks = c.k_row_scale[page, :, row].cpu().numpy()        # [L, H]
    vs = c.v_row_scale[page, :, row].cpu().numpy()
    return kc, vc, ks, vs


@pytest.mark.parametrize("dk,P", [(128, 16), (128, 32), (64, 16)])
def test_append_codes_and_row_scales_bit_exact(dk, P):
    w = W.custom(f"ra{dk}_{P}", 61, [37, 300, 1, 129], hq=16, hkv=2, dk=dk, dv=dk, page=P)
    st = State(w, "fp8", row_scales=True)
    for b in range(w.batch):
        kc, vc, ks, vs = _pool_rows(st, b)
        kc_ref, ks_ref = quant.quantize_rows(w.k_values(b).double().numpy())
        vc_ref, vs_ref = quant.quantize_rows(w.v_values(b).double().numpy())
        assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref), f"request {b} codes"
        assert np.array_equal(ks, ks_ref) and np.array_equal(vs, vs_ref), f"request {b} scales"


def _decode_check(w, split, requests=None):
    st = State(w, "fp8", split_tokens=split, row_scales=True)
    out = st.run().float().cpu().numpy()
    flags = step.flags(w)
    assert np.array_equal(st.step.abort.cpu().numpy(), flags)
    q = w.q_values().double().numpy()
    G = w.group
    for b in (range(w.batch) if requests is None else requests):
        if flags[b]:
            assert np.all(out[b] == 0.0)
            continue
        kc, ks = quant.quantize_rows(w.k_values(b).double().numpy())
        vc, vs = quant.quantize_rows(w.v_values(b).double().numpy())
        k = quant.dequantize_rows(kc, ks)
        v = quant.dequantize_rows(vc, vs)
        o_ref, _ = attention.attend(q[b], k, v, w.sm_scale)
        assert_close(out[b], o_ref, f"{w.name} request {b}")


@pytest.mark.parametrize("lens,P,split", [([300, 1000, 17, 513], 16, 128),
                                          ([1, 2, 31, 33, 64, 65], 16, 32),
                                          ([700, 129, 4000], 64, 1024),
                                          ([2048, 96], 32, 2048)])
def test_decode_over_row_scales(lens, P, split):
    """Ragged lengths (partial tiles read rows whose scales are unwritten and
    NaN), page sizes, splits of 1 to 128 pages."""
    w = W.custom(f"rd{len(lens)}_{P}", 62, lens, hq=64, hkv=8, dk=128, dv=128, page=P)
    _decode_check(w, split)


def test_decode_over_row_scales_aborted_and_small_groups():
    lens = [500, 1200, 64, 3000, 17, 900]
    w = W.custom("rab", 63, lens, hq=8, hkv=2, dk=128, dv=128, page=16, n_realloc=2)
    assert step.flags(w).any()
    _decode_check(w, 256)


def test_decode_sweep_b8_row_scales():
    _decode_check(W.sweep(8), None, requests=range(0, 8, 3))


def test_row_scales_unsupported_paths_refuse():
    w = W.custom("ru", 64, [100, 40], hq=16, hkv=2, dk=64, dv=64, page=16)
    st = State(w, "fp8", row_scales=True)
    with pytest.raises(pkv.PkvError):  # head dim 64: no decode kernel reads row scales
        st.run()
    w2 = W.custom("ru2", 65, [100, 40], hq=16, hkv=2, dk=128, dv=128, page=16)
    st2 = State(w2, "fp8", row_scales=True)
    q = torch.zeros((2, 2, 16, 128), dtype=torch.bfloat16, device=dev)
    o_part = torch.empty((2, 32, 1, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((2, 32, 1), dtype=torch.float32, device=dev)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_attn_drafts(st2.cache, q, st2.block_table, st2.seq_lens, 100, None,
                                   w2.sm_scale, 128, o_part, lse)


def test_decode_sweep_b16_row_scales():
    """Codes and row scales of the batch-16 sweep (about 600 MB) are read
    with non-temporal loads; the batch-8 case above reads plainly."""
    w = W.sweep(16)
    assert w.total_tokens * w.num_kv_heads * (2 * 128 + 8) > 384 << 20
    _decode_check(w, None, requests=[0, 15])


# ------------------------------------------------- range of the V row scales
def _row_case(v_amax, jump_log2, seed=71, L=300, hq=8, P=16, split=128):
    """One request whose K and V rows go through pkv_append with scales set
    at append. K rows are small (scores near 0) except token 200, aligned
    with query head 0 so that its score sits jump_log2 (log2 units) above the
    first tile's; V row t has largest magnitude v_amax[t % len(v_amax)].
    Returns (gpu out [hq, D], gpu lse [hq], oracle o, oracle lse, max |v|)."""
    D = 128
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((1, hq, D)).astype(np.float32)).to(torch.bfloat16)
    qd = q[0].double().numpy()
    sm = 1 / np.sqrt(D)
    k = rng.standard_normal((L, 1, D)) * 0.01
    if jump_log2:
        a = jump_log2 * np.log(2) / (sm * np.abs(qd[0]).sum())
        k[200, 0] = a * np.sign(qd[0])
    v = rng.standard_normal((L, 1, D))
    v /= np.abs(v).max(axis=2, keepdims=True)
    v *= np.asarray(v_amax, dtype=np.float64)[np.arange(L) % len(v_amax)][:, None, None]
    kb = torch.from_numpy(k.astype(np.float32)).to(torch.bfloat16)
    vb = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    n_pages = -(-L // P)
    cache = pkv.allocate_cache(n_pages + 3, 1, P, D, D, "fp8", device=dev, row_scales=True)
    perm = np.random.default_rng(seed + 1).permutation(n_pages + 3)[:n_pages].astype(np.int32)
    t = np.arange(L)
    slot = torch.from_numpy((perm[t // P] * P + t % P).astype(np.int32)).to(dev)
    pkv.pkv_append(cache, kb.to(dev), vb.to(dev), slot)
    bt = torch.from_numpy(perm[None, :]).to(dev)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    ds = pkv.DecodeStep(cache, hq, 1, L, split, verify=False)
    out = ds.attend(q.to(dev), bt, lens, sm, None).float().cpu().numpy()[0]
    lse = ds.lse.cpu().numpy()[0]
    kc, ks = quant.quantize_rows(kb.double().numpy())
    vc, vs = quant.quantize_rows(vb.double().numpy())
    o_ref, lse_ref = attention.attend(qd, quant.dequantize_rows(kc, ks),
                                      quant.dequantize_rows(vc, vs), sm)
    return out, lse, o_ref, lse_ref, float(np.max(np.abs(v_amax)))


@pytest.mark.parametrize("v_amax", [[1e-4], [1e4], [3e4, 1e-3], [1.0, 2.0, 0.5, 1000.0]],
                         ids=["small", "large", "mixed_large_small", "mixed"])
@pytest.mark.parametrize("jump", [0.0, 14.0], ids=["no_jump", "jump14"])
def test_decode_row_scales_extreme_v_ranges(v_amax, jump):
    """V rows of largest magnitude 1e-4 or 1e4 (scales far below and above
    1), alone or mixed within a tile, with or without a score 14 (log2)
    above the first tile's: the f16 numerators must neither overflow nor
    lose their precision. Judged relative to the largest value magnitude
    (the outputs of the small case are about 1e-5)."""
    out, lse, o_ref, lse_ref, vmax = _row_case(v_amax, jump)
    assert np.all(np.isfinite(out)), "non-finite output"
    err = np.abs(out - o_ref)
    tol = 2e-3 * vmax + 1e-2 * np.abs(o_ref)
    assert np.all(err <= tol), f"max err {err.max():.3e} (value scale {vmax:g})"
    assert np.all(np.abs(lse - lse_ref) <= 1e-3)


def test_append_rows_with_nan_and_infinity_match_the_oracle():
    """A NaN takes no part in its row's scale and becomes a NaN code with its
    sign; an infinite value makes the row's scale infinite (codes of the
    finite values are signed zeros, the infinity's code a NaN code)."""
    D, P = 128, 16
    rng = np.random.default_rng(72)
    x = rng.standard_normal((6, 2, D)).astype(np.float32)
    x[0, 0, 5] = np.nan
    x[1, 1, 0] = -np.nan
    x[1, 1, 100] = np.nan
    x[2, 0, :] = np.nan
    x[3, 1, 7] = np.inf
    x[4, 0, 9] = -np.inf
    xb = torch.from_numpy(x).to(torch.bfloat16)
    cache = pkv.allocate_cache(2, 2, P, D, D, "fp8", device=dev, row_scales=True)
    slot = torch.arange(6, dtype=torch.int32, device=dev)
    pkv.pkv_append(cache, xb.to(dev), xb.to(dev), slot)
    torch.cuda.synchronize()
    codes = cache.k_pool[0, :, :6, :].permute(1, 0, 2).cpu().numpy()
    scales = cache.k_row_scale[0, :, :6].permute(1, 0).cpu().numpy()
    c_ref, s_ref = quant.quantize_rows(xb.double().numpy())
    assert np.array_equal(np.isnan(scales), np.isnan(s_ref))
    ok = ~np.isnan(s_ref)
    assert np.array_equal(scales[ok], s_ref[ok])
    assert np.array_equal(codes, c_ref), np.argwhere(codes != c_ref)[:8].tolist()
