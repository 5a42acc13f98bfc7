"""The entry point that allocates nothing (pkv_decode_attn_static): decode
and combine with the split partials in the library's own device array.
Through the C ABI it must give the bits of the allocating pair
(pkv_decode_attn + pkv_combine with caller buffers) on the same inputs, on
two calls in a row whose second is smaller (the array keeps the first call's
partials), and refuse sizes beyond the array on the host."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from decode_attention_fp8_amd import _binding as B
from oracle import step
from tests.gpu_state import State, assert_close

pytestmark = pytest.mark.gpu


def test_scratch_size_matches_the_header():
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "pkv.h")).read()
    m = re.search(r"#define PKV_STATIC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == pkv.STATIC_SCRATCH_BYTES


def _allocating(st):
    """out, lse of the allocating pair on the State's inputs."""
    s = st.step
    pkv.pkv_verify(st.cache, st.block_table, st.expected, st.seq_lens, s.abort)
    pkv.pkv_decode_attn(st.cache, st.q, st.block_table, st.seq_lens, s.max_seq_len, s.abort,
                        st.w.sm_scale, s.split_tokens, s.o_part, s.lse_part)
    pkv.pkv_combine(s.o_part, s.lse_part, st.seq_lens, s.split_tokens, s.max_seq_len, s.abort,
                    s.out, s.lse)
    torch.cuda.synchronize()
    return s.out.clone(), s.lse.clone()


def _static(st):
    s = st.step
    out = torch.full_like(s.out, float("nan"))
    lse = torch.full_like(s.lse, float("nan"))
    pkv.pkv_verify(st.cache, st.block_table, st.expected, st.seq_lens, s.abort)
    pkv.pkv_decode_attn_static(st.cache, st.q, st.block_table, st.seq_lens, s.max_seq_len,
                               s.abort, st.w.sm_scale, s.split_tokens, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_two_calls_second_smaller_match_the_allocating_pair(kv):
    big = W.custom("na_big", 91, [3000, 1777, 4100, 65, 2500, 900], hq=64, hkv=8, dk=128,
                   dv=128, page=16, split=256, n_realloc=1)
    small = W.custom("na_small", 92, [300, 17], hq=16, hkv=2, dk=128, dv=128, page=16, split=128)
    for w in (big, small):
        st = State(w, kv)
        o_ref, l_ref = _allocating(st)
        o, l = _static(st)
        assert _same_bits(o, o_ref), f"{w.name}: output differs from the allocating pair"
        assert _same_bits(l, l_ref), f"{w.name}: lse differs from the allocating pair"
        # and both against the oracle on one request
        flags = step.flags(w)
        b = int(np.argmax(flags == 0))
        ks, vs = step.scales(w, kv)
        o_or, _ = step.request_output(w, b, kv, ks, vs, False)
        assert_close(o[b].float().cpu().numpy(), o_or, f"{w.name} request {b}")


def test_latent_shape_within_the_array():
    w = W.custom("na_lat", 93, [700, 64, 3000], hq=128, hkv=1, dk=576, dv=512, page=64,
                 latent=True, split=1024, sm_scale=1 / 24)
    st = State(w, "fp8")
    o_ref, l_ref = _allocating(st)
    o, l = _static(st)
    assert _same_bits(o, o_ref) and _same_bits(l, l_ref)


def test_sizes_beyond_the_array_are_refused_before_any_launch():
    w = W.custom("na_over", 94, [40], hq=64, hkv=8, dk=128, dv=128, page=16, split=16)
    st = State(w, "fp8")
    # batch 64 x 64 heads x 2048 splits x 129 x 4 bytes > 64 MiB
    B_, Hq = 64, 64
    q = torch.zeros((B_, Hq, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B_, 2048), dtype=torch.int32, device="cuda")
    lens = torch.ones(B_, dtype=torch.int32, device="cuda")
    out = torch.zeros((B_, Hq, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_attn_static(st.cache, q, bt, lens, 2048 * 16, None, 0.1, 16, out)
    assert e.value.status == pkv.PKV_EINVAL
    assert torch.all(out == 0)
