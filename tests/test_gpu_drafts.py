"""GPU parity of decode attention over a token and its drafts verified
together (pkv_decode_attn_drafts + pkv_combine) against the float64 oracle
(oracle.attention.attend_drafts over the dequantised cache), element by
element within |gpu - ref| <= 2e-3 + 1e-2 |ref|."""
import math

import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import attention, e4m3, step
from tests.gpu_state import State, assert_close

pytestmark = pytest.mark.gpu
dev = "cuda"


def _run_drafts(st, q, split, abort=None):
    w = st.w
    B, T, Hq, D = q.shape
    L = int(w.seq_lens.max())
    n_split = -(-L // split)
    o_part = torch.empty((B, T * Hq, n_split, D), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, T * Hq, n_split), dtype=torch.float32, device=dev)
    pkv.pkv_decode_attn_drafts(st.cache, q, st.block_table, st.seq_lens, L, abort, w.sm_scale,
                               split, o_part, lse_part)
    out = torch.empty((B, T * Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T * Hq), dtype=torch.float32, device=dev)
    pkv.pkv_combine(o_part, lse_part, st.seq_lens, split, L, abort, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().reshape(B, T, Hq, D), lse.cpu().numpy().reshape(B, T, Hq)


def _check(w, T, split, seed=0, requests=None, aborted=()):
    st = State(w, "fp8")
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((w.batch, T, w.num_q_heads, w.head_dim_k))
                         .astype(np.float32)).to(torch.bfloat16)
    abort = None
    if aborted:
        a = np.zeros(w.batch, dtype=np.uint8)
        a[list(aborted)] = 1
        abort = torch.from_numpy(a).to(dev)
    out, lse = _run_drafts(st, q.to(dev), split, abort)
    ks, vs = step.scales(w, "fp8")
    qd = q.double().numpy()
    for b in (range(w.batch) if requests is None else requests):
        if b in aborted:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        k, v = step.request_kv(w, b, "fp8", ks, vs)
        o_ref, lse_ref = attention.attend_drafts(qd[b], k, v, w.sm_scale)
        assert_close(out[b], o_ref, f"{w.name} T={T} request {b}")
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse[b]), fin)
        assert np.allclose(lse[b][fin], lse_ref[fin], atol=1e-3, rtol=1e-4)


def test_drafts_split_past_128_pages_is_unsupported():
    """A split's page ids are held in registers, 128 per unit: a 4096-token
    split at page 16 (256 pages) is refused before anything is launched."""
    w = W.custom("dr_long", 90, [5000, 300], hq=64, hkv=8, dk=128, dv=128, page=16)
    st = State(w, "fp8")
    q = torch.zeros((w.batch, 2, w.num_q_heads, w.head_dim_k), dtype=torch.bfloat16, device=dev)
    with pytest.raises(pkv.PkvError) as e:
        _run_drafts(st, q, 4096)
    assert e.value.status == pkv.PKV_EUNSUPPORTED
    _check(w, 2, 2048, requests=[0, 1])  # 128 pages: the limit itself runs


@pytest.mark.parametrize("T", [1, 2, 4])
def test_drafts_production_heads(T):
    """64 query / 8 kv heads: T x 8 <= 32 query rows per kv head."""
    w = W.custom("dr", 91, [300, 1000, 17, 513], hq=64, hkv=8, dk=128, dv=128, page=16)
    _check(w, T, 128)


@pytest.mark.parametrize("T,hq,hkv", [(5, 16, 2), (3, 4, 2), (8, 64, 8)])
def test_drafts_row_groups_and_group_sizes(T, hq, hkv):
    """More than 32 query rows per kv head (row groups), small groups."""
    w = W.custom("drg", 92, [200, 77, 640], hq=hq, hkv=hkv, dk=128, dv=128, page=16)
    _check(w, T, 64)


@pytest.mark.parametrize("T,hq,hkv", [(16, 64, 8), (40, 64, 8), (64, 64, 8)])
def test_drafts_many_row_groups_share_tiles(T, hq, hkv):
    """4, 10 and 16 row groups of 32 query rows per kv head: one workgroup of
    4 waves, then two workgroups of 8 (the second with idle waves that still
    load their share of every tile)."""
    w = W.custom(f"drm{T}", 95, [300, 129, 77], hq=hq, hkv=hkv, dk=128, dv=128, page=16)
    _check(w, T, 128)


@pytest.mark.parametrize("lens,P,split", [([1, 2, 3, 4], 16, 16), ([33, 31, 32, 47], 16, 32),
                                          ([129, 64, 65], 64, 64), ([4096 + 3], 32, 512),
                                          ([5000, 2049, 1100], 16, 2048)])
def test_drafts_ragged_lengths_splits_and_short_requests(lens, P, split):
    """Queries that see nothing (L < q_len), split boundaries inside the
    drafts (empty trailing splits for the first queries), page sizes, and
    128-page units (the second vector of page ids)."""
    w = W.custom(f"drr{len(lens)}_{P}", 93, lens, hq=16, hkv=2, dk=128, dv=128, page=P)
    _check(w, 4, split)


def test_drafts_aborted_requests_write_zeros():
    w = W.custom("dra", 94, [300, 80, 500], hq=32, hkv=4, dk=128, dv=128, page=16)
    _check(w, 3, 128, aborted=(1,))


def test_drafts_score_jump_rescales():
    """Keys of a late page aligned with one query row's query: that row's
    score leaps far above the reference max set by earlier tiles."""
    hq, hkv, D, P, L, T = 8, 1, 128, 16, 256, 4
    rng = np.random.default_rng(95)
    q = rng.standard_normal((1, T, hq, D)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    sign = np.sign(qb[0, 2, 3].float().numpy())
    sign[sign == 0] = 1
    vals_k = rng.standard_normal((L, D)).astype(np.float32) * 0.01
    vals_k[160:176] = 7.0 * sign
    vals_v = rng.standard_normal((L, D)).astype(np.float32)
    ks = np.float32(np.abs(vals_k).max() / 448.0)
    vs = np.float32(np.abs(vals_v).max() / 448.0)
    kc = e4m3.encode((vals_k / ks).astype(np.float32))
    vc = e4m3.encode((vals_v / vs).astype(np.float32))
    cache = pkv.allocate_cache(L // P, hkv, P, D, D, "fp8", device=dev)
    cache.k_scale.fill_(float(ks))
    cache.v_scale.fill_(float(vs))
    cache.k_pool[:, 0] = torch.from_numpy(kc.reshape(L // P, P, D)).to(dev)
    cache.v_pool[:, 0] = torch.from_numpy(vc.reshape(L // P, P, D)).to(dev)

    class _St:
        pass
    st = _St()
    st.w = W.custom("drj", 96, [L], hq=hq, hkv=hkv, dk=D, dv=D, page=P)
    st.cache = cache
    st.block_table = torch.arange(L // P, dtype=torch.int32, device=dev).view(1, -1)
    st.seq_lens = torch.tensor([L], dtype=torch.int32, device=dev)
    out, _ = _run_drafts(st, qb.to(dev), 256)
    k_hat = (e4m3.DECODE[kc] * np.float64(ks))[:, None, :]
    v_hat = (e4m3.DECODE[vc] * np.float64(vs))[:, None, :]
    o_ref, _ = attention.attend_drafts(qb[0].double().numpy(), k_hat, v_hat, st.w.sm_scale)
    assert_close(out[0], o_ref, "drafts score jump")


def test_drafts_footprint_above_cache_sampled():
    """The batch-16 sweep cache (285,175 tokens, 584 MB of codes) is read with
    non-temporal loads, the small caches above with plain ones: three
    requests of a q_len-4 launch."""
    w = W.sweep(16)
    assert w.total_tokens * w.num_kv_heads * 2 * 128 > 384 << 20
    _check(w, 4, 1024, seed=5, requests=[0, 9, 15])
