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
