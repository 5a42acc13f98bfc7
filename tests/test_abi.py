"""CPU checks of the C-ABI boundary: the library loads, exports every
function include/pkv.h declares, and rejects bad arguments on the host
before anything reaches a GPU (no compute calls here)."""
import ctypes
import os
import re

import torch
import subprocess

import pytest

import decode_attention_fp8_amd as pkv
from decode_attention_fp8_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", src)))


def test_header_declares_the_four_hot_path_calls():
    d = declared()
    for name in ("pkv_append", "pkv_verify", "pkv_decode_attn", "pkv_combine"):
        assert name in d


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pkv_\w+)", nm))
    assert set(declared()) <= exported
    assert set(B.EXPORTS) == set(declared())


def test_host_helpers():
    assert pkv.pkv_version() >= 100
    assert pkv.pkv_strerror(0) == "ok"
    assert pkv.pkv_strerror(-1) == "invalid argument"
    # geometry only: one-page host tensors stand in for the pools
    gqa = pkv.Cache(torch.empty((1, 8, 16, 128), dtype=torch.uint8),
                    torch.empty((1, 8, 16, 128), dtype=torch.uint8))
    # batch 64 of the concurrency sweep: long splits; batch 1: short ones
    assert pkv.pkv_suggest_split(gqa, 64, 64, 64 * 17000, 32768) == 2048
    gqa_bf16 = pkv.Cache(torch.empty((1, 8, 16, 128), dtype=torch.bfloat16),
                         torch.empty((1, 8, 16, 128), dtype=torch.bfloat16))
    assert pkv.pkv_suggest_split(gqa_bf16, 64, 64, 64 * 17000, 32768) == 2048
    assert pkv.pkv_suggest_split(gqa, 64, 8, 8 * 17000, 32768) == 512
    assert pkv.pkv_suggest_split(gqa, 64, 1, 17000, 17000) == 128
    # batch 8 x 4096: 256-token splits still give 1064 units, so not 128
    assert pkv.pkv_suggest_split(gqa, 64, 8, 8 * 4096, 4096) == 256
    # never longer than the longest request (rounded up to whole pages)
    assert pkv.pkv_suggest_split(gqa, 64, 1, 10, 10) == 16
    lat = pkv.Cache(torch.empty((1, 1, 64, 576), dtype=torch.uint8), None, latent_dim_v=512)
    # latent: about an eighth of an equal per-compute-unit share of the pages
    assert pkv.pkv_suggest_split(lat, 128, 64, 907520, 65536) == 128
    assert pkv.pkv_suggest_split(lat, 128, 1, 8192, 8192) == 64
    for s in (pkv.pkv_suggest_split(gqa, 64, 3, 0, 5000), pkv.pkv_suggest_split(lat, 128, 3, 0, 5000)):
        assert s > 0 and s % 16 == 0
    # the step in two launches: grouped-query head dim 128, static scales or
    # bf16, up to 128 pages per split
    assert pkv.pkv_step_launches(gqa, 64, 2048) == 2
    assert pkv.pkv_step_launches(gqa_bf16, 64, 256) == 2
    assert pkv.pkv_step_launches(gqa, 64, 4096) == 3
    assert pkv.pkv_step_launches(gqa, 8, 2048) == 2 and pkv.pkv_step_launches(gqa, 256, 2048) == 3
    assert pkv.pkv_step_launches(lat, 128, 256) == 3
    d64 = pkv.Cache(torch.empty((1, 2, 16, 64), dtype=torch.uint8),
                    torch.empty((1, 2, 16, 64), dtype=torch.uint8))
    assert pkv.pkv_step_launches(d64, 8, 64) == 3
    with pytest.raises(pkv.PkvError):
        pkv.pkv_suggest_split(gqa, 63, 1, 10, 10)  # query heads not a multiple of kv heads
    with pytest.raises(pkv.PkvError):
        pkv.pkv_suggest_split(gqa, 64, 0, 10, 10)


def _cache(**kw):
    base = dict(k_pool=16, v_pool=32, dtype=1, num_pages=4, page_size=16, num_kv_heads=1,
                head_dim_k=64, head_dim_v=64, k_scale=48, v_scale=64, page_tags=80)
    base.update(kw)
    return B.PkvCacheStruct(**base)


def test_invalid_arguments_rejected_on_host():
    lib = B._lib
    E = B.PKV_EINVAL
    P = 4096  # a fake, aligned, never-dereferenced address
    # scales
    assert lib.pkv_scales_from_amax(None, 1, 1, 64, 0, P, None) == E
    assert lib.pkv_scales_from_amax(P, 1, 1, 60, 0, P, None) == E
    assert lib.pkv_scales_from_amax(P + 2, 1, 1, 64, 0, P, None) == E
    # append
    assert lib.pkv_append(None, P, P, P, None, None, 1, None) == E
    assert lib.pkv_append(ctypes.byref(_cache(page_size=24)), P, P, P, None, None, 1, None) == E
    assert lib.pkv_append(ctypes.byref(_cache(head_dim_k=72)), P, P, P, None, None, 1, None) == E
    assert lib.pkv_append(ctypes.byref(_cache(v_pool=None)), P, P, P, None, None, 1, None) == E
    assert lib.pkv_append(ctypes.byref(_cache()), P, None, P, None, None, 1, None) == E
    assert lib.pkv_append(ctypes.byref(_cache(k_scale=None)), P, P, P, None, None, 1, None) == E
    # verify
    assert lib.pkv_verify(ctypes.byref(_cache(page_tags=None)), P, P, P, 1, 1, P, None) == E
    assert lib.pkv_verify(ctypes.byref(_cache()), P, P, P, -1, 1, P, None) == E
    assert lib.pkv_verify(ctypes.byref(_cache()), P, P, P, 1, 0, P, None) == E
    # decode: split not a page multiple, q heads not a kv multiple, bounds inconsistent
    c = ctypes.byref(_cache(num_kv_heads=2))
    assert lib.pkv_decode_attn(c, P, 8, P, P, 1, 4, 64, None, 0.1, 24, 8, P, P, None) == E
    assert lib.pkv_decode_attn(c, P, 7, P, P, 1, 4, 64, None, 0.1, 16, 8, P, P, None) == E
    assert lib.pkv_decode_attn(c, P, 8, P, P, 1, 4, 65, None, 0.1, 16, 8, P, P, None) == E
    assert lib.pkv_decode_attn(c, P, 8, P, P, 1, 4, 64, None, 0.1, 16, 3, P, P, None) == E
    assert lib.pkv_decode_attn(c, None, 8, P, P, 1, 4, 64, None, 0.1, 16, 8, P, P, None) == E
    # decode: unsupported shapes
    U = B.PKV_EUNSUPPORTED
    assert lib.pkv_decode_attn(ctypes.byref(_cache(head_dim_k=96, head_dim_v=96)), P, 1, P, P, 1,
                               4, 64, None, 0.1, 16, 8, P, P, None) == U
    assert lib.pkv_decode_attn(ctypes.byref(_cache(num_kv_heads=1)), P, 3, P, P, 1, 4, 64, None,
                               0.1, 16, 8, P, P, None) == U
    # combine
    assert lib.pkv_combine(None, P, P, 1, 1, 64, 16, 4, 64, None, P, None, None) == E
    assert lib.pkv_combine(P, P, P, 1, 1, 64, 16, 3, 64, None, P, None, None) == E
    assert lib.pkv_combine(P, P, P, 1, 1, 60, 16, 4, 64, None, P, None, None) == E
    # the step in two calls: every argument is checked before any launch
    sd, sc = lib.pkv_step_decode, lib.pkv_step_combine
    g = ctypes.byref(_cache(num_kv_heads=2, head_dim_k=128, head_dim_v=128))
    ok = (P, 8, P, P, P, P, P, 1, 4, 64, 0.1, 16, 8, P, P, P, P, None)
    assert sd(ctypes.byref(_cache(page_tags=None)), *ok) == E
    assert sd(g, *ok[:15], None, *ok[16:]) == E              # unit_flags
    assert sd(g, *ok[:16], None, None) == E                  # abort_out
    assert sd(g, P, 8, P + 2, *ok[3:]) == E                   # k_new misaligned
    assert sd(g, P, 8, P, None, *ok[4:]) == E                 # v_new missing (separate pools)
    assert sd(g, *ok[:11], 24, *ok[12:]) == E                 # split not a page multiple
    assert sd(g, *ok[:12], 3, *ok[13:]) == E                  # max_splits too small
    assert sd(g, None, *ok[1:]) == E                          # q
    okc = (8, P, P, P, P, P, 1, 4, 64, 16, 8, P, P, P, P, P, None, None)
    assert sc(g, *okc[:13], None, *okc[14:]) == E             # unit_flags
    assert sc(g, *okc[:14], None, *okc[15:]) == E             # abort_out
    assert sc(g, 8, P, P, None, *okc[4:]) == E                # block_table
    assert sc(ctypes.byref(_cache(page_tags=None)), *okc) == E
    # INT4 linear: NULL, batch outside [1, 64], n not a multiple of 32, k not a
    # multiple of 1024, misaligned pointers (the workspace too)
    assert lib.pkv_int4_linear(None, P, P, 1, 32, 1024, P, None, None) == E
    assert lib.pkv_int4_linear(P, P, P, 0, 32, 1024, P, None, None) == E
    assert lib.pkv_int4_linear(P, P, P, 65, 32, 1024, P, None, None) == E
    assert lib.pkv_int4_linear(P, P, P, 1, 48, 1024, P, None, None) == E
    assert lib.pkv_int4_linear(P, P, P, 1, 32, 1536, P, None, None) == E
    assert lib.pkv_int4_linear(P + 8, P, P, 1, 32, 1024, P, None, None) == E
    assert lib.pkv_int4_linear(P, P, P, 16, 8192, 8192, P, P + 4, None) == E
    # workspace: none up to 8 tokens or when the row blocks fill the chip; above,
    # one fp32 partial per input slice (8192 rows: 64 blocks of 128, 4 slices)
    ws = lib.pkv_int4_linear_workspace
    assert ws(8, 8192, 8192) == 0
    assert ws(16, 8192, 8192) == 4 * 16 * 8192 * 4
    assert ws(64, 8192, 8192) == 4 * 64 * 8192 * 4
    assert ws(64, 28672, 8192) == 0
    assert ws(9, 128, 2048) == 8 * 9 * 128 * 4
    assert ws(33, 96, 2048) == 0          # rows not a multiple of 128: no split
    assert ws(0, 8192, 8192) == E and ws(65, 8192, 8192) == E


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pkv.pkv_scales_from_amax(x, False, torch.zeros(1))
