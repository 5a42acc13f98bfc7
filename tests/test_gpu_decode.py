"""GPU parity of the decode path (verify -> append -> decode -> combine)
against the float64 oracle, element by element on sampled requests and
heads, within |gpu - ref| <= 2e-3 + 1e-2 |ref|."""
import math

import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import e4m3, step
from tests.gpu_state import State, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu
dev = "cuda"


def _check_requests(st, requests, kv_heads=None, kv_dtype=None):
    """Output rows and lse of the sampled requests and kv heads' query heads
    against the oracle; aborted requests must give exactly 0 and -inf."""
    w = st.w
    kv_dtype = kv_dtype or st.kv_dtype
    out = st.run().float().cpu().numpy()
    lse = st.step.lse.cpu().numpy()
    ks, vs = step.scales(w, kv_dtype)
    flags = step.flags(w)
    assert np.array_equal(st.step.abort.cpu().numpy(), flags)
    q = w.q_values().double().numpy()
    G = w.group
    hs = np.arange(w.num_kv_heads) if kv_heads is None else np.asarray(kv_heads)
    qh = np.concatenate([np.arange(h * G, (h + 1) * G) for h in hs])
    for b in requests:
        o_ref, lse_ref = step.request_output(w, b, kv_dtype, ks, vs, bool(flags[b]), hs, q[b])
        got = out[b][qh]
        if flags[b]:
            assert np.all(got == 0.0), f"aborted request {b} must be zero"
            assert np.all(np.isneginf(lse[b][qh])), f"aborted request {b} lse must be -inf"
        else:
            assert_close(got, o_ref, f"{w.name} {kv_dtype} request {b}")
            assert_lse_close(lse[b][qh], lse_ref, f"{w.name} {kv_dtype} request {b} lse")
    return out


def _zero_query_sentinel(st):
    """With q = 0 every score is 0: each weight is 1 / L_b, so lse = ln L_b
    and out = the mean of the request's values. The denominators count
    tokens exactly, so a tile lost or read twice anywhere in the launch moves
    lse by about 32 / L_b (2e-3 at 16k tokens), far outside 1e-5."""
    w = st.w
    st.q.zero_()
    st.run()
    lse = st.step.lse.cpu().numpy().astype(np.float64)
    flags = step.flags(w)
    for b in range(w.batch):
        if flags[b]:
            assert np.all(np.isneginf(lse[b]))
        else:
            err = np.abs(lse[b] - math.log(int(w.seq_lens[b])))
            assert err.max() <= 1e-5, f"{w.name} request {b}: lse off ln L by {err.max():.2e}"
    return flags


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_tiny(kv):
    st = State(W.tiny(), kv)
    out = _check_requests(st, [0, 1])
    assert st.step.abort.cpu().tolist() == [0, 1]
    assert np.all(out[1] == 0)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_tiny_unused_page_bump_aborts_nothing(kv):
    st = State(W.tiny(bump_unused=True), kv)
    _check_requests(st, [0, 1])
    assert st.step.abort.cpu().tolist() == [0, 0]


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_gqa_batch8_ctx4096(kv):
    st = State(W.gqa(), kv)
    _check_requests(st, [0, 5])


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_sweep_b8(kv):
    st = State(W.sweep(8), kv)
    _check_requests(st, [2, 7], kv_heads=[0, 5])


def test_sweep_b64_full_size_sampled():
    st = State(W.sweep(64), "fp8")
    _check_requests(st, [0, 31, 63], kv_heads=[3])


@pytest.mark.parametrize("B", [1, 16, 32])
def test_sweep_other_batches_sampled(B):
    st = State(W.sweep(B), "fp8")
    reqs = sorted({0, B // 2, B - 1})
    _check_requests(st, reqs, kv_heads=[0, 7] if B == 1 else [5])


@pytest.mark.parametrize("make", [lambda: W.sweep(64), W.long_context],
                         ids=["sweep_b64", "long_b4"])
def test_bf16_cache_at_the_sizes_timed(make):
    """The bf16-cache comparison runs at the sizes the measurement times."""
    w = make()
    st = State(w, "bf16")
    _check_requests(st, [0, w.batch - 1], kv_heads=[2])


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("make", [lambda: W.sweep(64), W.long_context, W.mla],
                         ids=["sweep_b64", "long_b4", "mla_b64"])
def test_zero_query_sentinel_full_size(make, kv):
    """Every (request, head) of the full workload at once: lse must be ln L_b
    to 1e-5 (and the output the mean value row, checked on one request)."""
    w = make()
    st = State(w, kv)
    flags = _zero_query_sentinel(st)
    b = int(np.argmin(np.where(flags == 0, w.seq_lens, np.iinfo(np.int32).max)))
    ks, vs = step.scales(w, kv)
    _, v = step.request_kv(w, b, kv, ks, vs, heads=[0])
    mean = v[:, 0, :].mean(axis=0)
    got = st.step.out[b, :w.group].float().cpu().numpy()
    assert_close(got, np.broadcast_to(mean, got.shape), f"{w.name} {kv} zero query, request {b}")


def test_short_splits_on_long_ragged_requests():
    """Splits of 128 tokens on 8 long requests (up to 128 partials each for
    the combine): ragged lengths, one request shorter than a split; every
    request, two kv heads."""
    lens = [16384, 16307, 16000, 15999, 130, 16384, 9000, 16383]
    w = W.custom("units2", 77, lens, hq=64, hkv=8, dk=128, dv=128, page=16, split=128)
    st = State(w, "fp8")
    assert st.step.split_tokens == 128
    _check_requests(st, list(range(8)), kv_heads=[0, 7])


def test_pages_past_4gib_of_pool():
    """Four requests' pages scattered over a 600,000-page pool (9.8 GB per
    pool): about half of them start past 4 GiB, so every page offset takes
    64 bits. Every request, two kv heads."""
    w = W.custom("bigpool", 88, [2000, 1500, 777, 3000], hq=64, hkv=8, dk=128, dv=128,
                 page=16, pool_pages=600000)
    page_bytes = 8 * 16 * 128
    assert int(w.block_table.max()) * page_bytes > 2 ** 32
    st = State(w, "fp8")
    _check_requests(st, [0, 1, 2, 3], kv_heads=[0, 7])
    del st
    torch.cuda.empty_cache()


def test_long_context_split256_sampled():
    st = State(W.long_context(), "fp8")
    assert st.step.split_tokens == 256 and st.step.max_splits == 512
    _check_requests(st, [2], kv_heads=[6])


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_mla_sampled_including_aborted(kv):
    w = W.mla()
    st = State(w, kv)
    flags = step.flags(w)
    aborted = [int(np.nonzero(flags)[0][0])]
    shortest = [int(np.argmin(w.seq_lens))]
    longest = [int(np.argmax(np.where(flags == 0, w.seq_lens, 0)))]
    _check_requests(st, sorted(set(aborted + shortest + longest)))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("hq,lens,split", [(64, [1, 63, 64, 65, 700], 64), (128, [129, 2000], 512),
                                           (128, [4100, 33], 1024), (256, [700, 64, 3000], 2048)])
def test_mla_shapes_ragged(kv, hq, lens, split):
    w = W.custom(f"mla{hq}", 81, lens, hq=hq, hkv=1, dk=576, dv=512, page=64, latent=True,
                 split=split, sm_scale=1 / math.sqrt(576))
    st = State(w, kv)
    _check_requests(st, range(w.batch))


# ------------------------------------------------------------- edge cases
@pytest.mark.parametrize("lens,P,split", [([1], 16, 16), ([16, 17, 15], 16, 16), ([1, 2, 3, 4], 64, 64),
                                          ([300, 1, 257], 32, 96), ([5000, 33], 16, 256),
                                          ([2100, 1024, 1023, 47], 16, 1024),
                                          ([4096 + 640, 4096, 65], 64, 4096),
                                          ([70, 33, 80], 16, 32)])
@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_ragged_lengths_and_splits(lens, P, split, kv):
    w = W.custom(f"rag{len(lens)}_{P}", 77, lens, hq=8, hkv=2, dk=128, dv=128, page=P, split=split)
    st = State(w, kv)
    _check_requests(st, range(w.batch))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("G,dk", [(1, 64), (1, 128), (2, 128), (16, 128), (4, 64)])
def test_group_sizes_and_head_dims(G, dk, kv):
    w = W.custom(f"g{G}", 78, [77, 513], hq=2 * G, hkv=2, dk=dk, dv=dk, page=16)
    st = State(w, kv)
    _check_requests(st, range(w.batch))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("shape", [dict(hq=4, hkv=1, dk=64, dv=64, page=16),
                                   dict(hq=8, hkv=1, dk=128, dv=128, page=16),
                                   dict(hq=128, hkv=1, dk=576, dv=512, page=64, latent=True)],
                         ids=["generic", "grouped_query", "latent"])
@pytest.mark.parametrize("empty", [[1], [0, 1, 2]], ids=["one_empty", "all_empty"])
def test_empty_request_gives_zero_and_neg_inf_lse(shape, empty, kv):
    """Requests of length 0 give exactly 0 and lse = -inf; the others still
    match the oracle. With every request empty the latent kernel's launch
    has no tiles at all."""
    w = W.custom("e", 79, [40, 130, 70], **shape)
    st = State(w, kv)
    for b in empty:
        st.seq_lens[b] = 0
    out = st.step.run(st.q, st.block_table, st.expected, st.seq_lens, w.sm_scale)
    torch.cuda.synchronize()
    for b in empty:
        assert torch.all(out[b] == 0)
        assert torch.all(torch.isneginf(st.step.lse[b]))
    rest = [b for b in range(w.batch) if b not in empty]
    if rest:
        ks, vs = step.scales(w, kv)
        q = w.q_values().double().numpy()
        got = out.float().cpu().numpy()
        for b in rest:
            o_ref, _ = step.request_output(w, b, kv, ks, vs, False, np.arange(w.num_kv_heads), q[b])
            assert_close(got[b], o_ref, f"empty-neighbour request {b}")


def test_every_e4m3_code_decodes_exactly():
    """Single-token requests over rows written directly with every code:
    the output is that token's value row, so it must be bf16(decode * s)."""
    s = np.float32(0.75)
    n_tok = 4
    cache = pkv.allocate_cache(n_tok, 1, 16, 64, 64, "fp8", device=dev)
    cache.k_scale.fill_(float(s))
    cache.v_scale.fill_(float(s))
    codes = np.arange(256, dtype=np.uint8).reshape(n_tok, 64)
    for i in range(n_tok):
        cache.k_pool[i, 0, 0, :] = 0x38  # key 1.0 everywhere (any finite key works)
        cache.v_pool[i, 0, 0, :] = torch.from_numpy(codes[i]).to(dev)
    bt = torch.arange(n_tok, dtype=torch.int32, device=dev).view(n_tok, 1)
    lens = torch.ones(n_tok, dtype=torch.int32, device=dev)
    q = torch.ones((n_tok, 1, 64), dtype=torch.bfloat16, device=dev)
    ds = pkv.DecodeStep(cache, 1, n_tok, 1, 16, verify=False)
    out = ds.attend(q, bt, lens, 0.125, None).float().cpu().numpy()[:, 0, :]
    ref = (e4m3.DECODE[codes] * np.float64(s)).astype(np.float32)
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    assert np.array_equal(np.isnan(out), np.isnan(ref_bf16))
    ok = ~np.isnan(ref_bf16)
    assert np.array_equal(out[ok], ref_bf16[ok])


@pytest.mark.parametrize("kv_nan", [False, True], ids=["finite_codes", "nan_code"])
def test_latent_every_e4m3_code_exact(kv_nan):
    """The 128-head e4m3 latent kernel multiplies V's codes as they are (fp8
    MFMA). Single-token requests (weight exactly 1, q = 0) whose V rows hold
    every finite code: each output must be bf16(decode(code) * s) for every
    head, bit for bit. With a NaN code in the row, the score (V is the row's
    first 512 values) and every output of the request are NaN."""
    hq, dk, dv, P = 128, 576, 512, 64
    s = np.float32(0.375)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)  # 254 codes
    n_req = 3
    rows = np.full((n_req, dk), 0x38, dtype=np.uint8)
    for i in range(n_req):
        rows[i, :dv] = np.roll(np.resize(finite, dv), 97 * i)
    if kv_nan:
        rows[1, 300] = 0xFF
    cache = pkv.allocate_cache(n_req, 1, P, dk, dv, "fp8", latent=True, device=dev)
    cache.k_pool[:, 0, 0, :] = torch.from_numpy(rows).to(dev)
    cache.k_scale.fill_(float(s))
    cache.v_scale = cache.k_scale
    bt = torch.arange(n_req, dtype=torch.int32, device=dev).view(n_req, 1)
    lens = torch.ones(n_req, dtype=torch.int32, device=dev)
    q = torch.zeros((n_req, hq, dk), dtype=torch.bfloat16, device=dev)
    ds = pkv.DecodeStep(cache, hq, n_req, 1, 64, verify=False)
    out = ds.attend(q, bt, lens, 1 / math.sqrt(dk), None).float().cpu().numpy()
    ref = (e4m3.DECODE[rows[:, :dv]] * np.float64(s)).astype(np.float32)
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    for i in range(n_req):
        if kv_nan and i == 1:
            assert np.all(np.isnan(out[i])), "a NaN code makes the request's outputs NaN"
        else:
            assert np.array_equal(out[i], np.broadcast_to(ref_bf16[i], (hq, dv))), f"request {i}"


@pytest.mark.parametrize("nan_tokens", [(37,), (37, 80)], ids=["one_split", "every_split"])
def test_nan_key_code_gives_nan_rows(nan_tokens):
    """A NaN code in a key makes that token's score NaN for every query head
    of its kv head, and so their outputs and lse (as the oracle's max and
    exp do), whether the NaN sits in one of the request's two splits or in
    both; the other kv head is untouched."""
    from oracle import attention
    hq, hkv, D, P, L, split = 16, 2, 128, 16, 100, 64
    n_pages = -(-L // P)
    rng = np.random.default_rng(41)
    vals = rng.standard_normal((2, n_pages * P, hkv, D)).astype(np.float32)
    cache = pkv.allocate_cache(n_pages, hkv, P, D, D, "fp8", device=dev)
    hat = []
    for x, pool, scale in ((vals[0], cache.k_pool, cache.k_scale), (vals[1], cache.v_pool, cache.v_scale)):
        sc = (np.abs(x).max(axis=(0, 2)) / 448.0).astype(np.float32)
        codes = e4m3.encode((x / sc[None, :, None]).astype(np.float32))
        if pool is cache.k_pool:
            for t in nan_tokens:
                codes[t, 1, 5] = 0x7F
        hat.append(e4m3.DECODE[codes] * sc[None, :, None].astype(np.float64))
        pool[:] = torch.from_numpy(codes.reshape(n_pages, P, hkv, D).transpose(0, 2, 1, 3).copy()).to(dev)
        scale.copy_(torch.from_numpy(sc).to(dev))
    q = torch.from_numpy(rng.standard_normal((1, hq, D)).astype(np.float32)).to(torch.bfloat16)
    bt = torch.arange(n_pages, dtype=torch.int32, device=dev).view(1, n_pages)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    sm = 1 / math.sqrt(D)
    ds = pkv.DecodeStep(cache, hq, 1, L, split, verify=False)
    out = ds.attend(q.to(dev), bt, lens, sm, None).float().cpu().numpy()[0]
    lse = ds.lse.cpu().numpy()[0]
    ref, lse_ref = attention.attend(q[0].double().numpy(), hat[0][:L], hat[1][:L], sm)
    assert np.all(np.isnan(ref[8:])) and np.all(np.isnan(lse_ref[8:]))
    assert np.all(np.isnan(out[8:])), "kv head 1's query heads must be NaN"
    assert np.all(np.isnan(lse[8:]))
    assert_close(out[:8], ref[:8], "kv head 0")
    assert_lse_close(lse[:8], lse_ref[:8], "kv head 0 lse")


def test_noop_tracker_equals_checked_path_when_nothing_aborts():
    w = W.gqa(2, 1000)
    a = State(w, "fp8", verify=True).run().clone()
    b = State(w, "fp8", verify=False).run().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_deterministic_bitwise():
    st = State(W.sweep(8), "fp8")
    a = st.run().clone()
    b = st.run().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_split_size_does_not_change_the_result_beyond_rounding():
    w = W.custom("sp", 80, [3000, 1777], hq=16, hkv=2, dk=128, dv=128, page=16)
    outs = [State(w, "fp8", split_tokens=s).run().float().cpu().numpy() for s in (16, 256, 3008)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 4e-3


def test_fp8_close_to_bf16_reported():
    """FP8 against BF16 attention on the same inputs: not a pinned quantity
    (the pages' evidence is model-level accuracy); only sanity-bounded."""
    w = W.gqa(2, 2048)
    a = State(w, "fp8").run().float()
    b = State(w, "bf16").run().float()
    err = (a - b).abs().max().item()
    assert math.isfinite(err) and err < 0.1


@pytest.mark.parametrize("make", [W.tiny, lambda: W.sweep(8)])
def test_graph_replays_match_eager_step(make):
    """The step captured as a HIP graph and replayed (with eager work and
    synchronisation between replays) gives the eager step's bits every time."""
    w = make()
    st = State(w, "fp8")
    args = (st.q, st.block_table, st.expected, st.seq_lens, w.sm_scale, st.new_k, st.new_v,
            st.new_slot, st.new_req)
    eager = st.step.run(*args).clone()
    eager_lse = st.step.lse.clone()
    eager_abort = st.step.abort.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step.run(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step.run(*args)
    for _ in range(3):
        st.step.out.zero_()
        st.step.lse.fill_(1.0)
        st.step.abort.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.step.out.view(torch.int16), eager.view(torch.int16))
        assert torch.equal(st.step.lse.view(torch.int32), eager_lse.view(torch.int32))
        assert torch.equal(st.step.abort, eager_abort)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_mla_score_jump_far_above_the_first_tile(kv):
    """Keys of a later page aligned with head 0's query push its score about
    190 (log2 units) above every score of the first page: the running max
    must move (or the unit restart) without losing accuracy."""
    from oracle import attention
    hq, dk, dv, P, L = 128, 576, 512, 64, 256
    rng = np.random.default_rng(9)
    q = torch.from_numpy(rng.standard_normal((1, hq, dk)).astype(np.float32)).to(torch.bfloat16)
    sign = np.sign(q[0, 0].float().numpy())
    sign[sign == 0] = 1
    vals = rng.standard_normal((L, dk)).astype(np.float32) * 0.01   # small keys ...
    vals[128:192] = 7.0 * sign                                        # ... except page 2
    scale = np.float32(7.0 / 448.0)
    cache = pkv.allocate_cache(4, 1, P, dk, dv, kv, latent=True, device=dev)
    if kv == "fp8":
        codes = e4m3.encode((vals / scale).astype(np.float32))
        k_hat = e4m3.DECODE[codes] * np.float64(scale)
        cache.k_pool[:, 0] = torch.from_numpy(codes.reshape(4, P, dk)).to(dev)
        cache.k_scale.fill_(float(scale))
        cache.v_scale = cache.k_scale
    else:
        kb = torch.from_numpy(vals).to(torch.bfloat16)
        k_hat = kb.double().numpy()
        cache.k_pool[:, 0] = kb.view(4, P, dk).to(dev)
    bt = torch.arange(4, dtype=torch.int32, device=dev).view(1, 4)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    sm = 1 / math.sqrt(dk)
    ds = pkv.DecodeStep(cache, hq, 1, L, 256, verify=False)
    out = ds.attend(q.to(dev), bt, lens, sm, None).float().cpu().numpy()[0]
    ref, _ = attention.attend(q[0].double().numpy(), k_hat[:, None, :], k_hat[:, None, :dv], sm)
    assert_close(out, ref, f"mla score jump {kv}")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_mla_huge_context_chunks_zero_query(kv):
    """One request of 8,400,037 tokens (131,251 pages of 64, 4.8 GB as e4m3):
    the 128-head latent kernel's equal shares then exceed 512 tiles, so a
    segment is taken in several chunks of page ids. Every row of page p is
    one of seven random patterns (p mod 7). With q = 0 every score is 0, so
    the output is the mean of the rows' first 512 values, a closed form over
    the patterns' token counts, and lse = ln L; a dropped or doubled tile
    moves both."""
    hq, dk, dv, P, L = 128, 576, 512, 64, 8_400_037
    n_pages = -(-L // P)
    rng = np.random.default_rng(23)
    cache = pkv.allocate_cache(n_pages, 1, P, dk, dv, kv, latent=True, device=dev, poison=False)
    which = torch.arange(n_pages, device=dev) % 7
    if kv == "fp8":
        pat = rng.integers(0, 256, size=(7, dk), dtype=np.uint8)
        pat[(pat & 0x7F) == 0x7F] = 0x38                      # no NaN codes
        scale = np.float32(0.25)
        vals = e4m3.DECODE[pat] * np.float64(scale)
        cache.k_pool.view(n_pages, P, dk)[:] = torch.from_numpy(pat).to(dev)[which][:, None, :]
        cache.k_scale.fill_(float(scale))
        cache.v_scale = cache.k_scale
    else:
        pat = torch.from_numpy(rng.standard_normal((7, dk)).astype(np.float32)).to(torch.bfloat16)
        vals = pat.double().numpy()
        cache.k_pool.view(n_pages, P, dk)[:] = pat.to(dev)[which][:, None, :]
    # tokens per pattern: whole pages, then the last page's L - P (n_pages - 1)
    counts = np.bincount(np.arange(n_pages) % 7, minlength=7).astype(np.float64) * P
    counts[(n_pages - 1) % 7] -= n_pages * P - L
    ref = (counts[:, None] * vals[:, :dv]).sum(axis=0) / L
    bt = torch.arange(n_pages, dtype=torch.int32, device=dev).view(1, n_pages)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    split = pkv.pkv_suggest_split(cache, hq, 1, L, L)
    ds = pkv.DecodeStep(cache, hq, 1, L, split, verify=False)
    q = torch.zeros((1, hq, dk), dtype=torch.bfloat16, device=dev)
    out = ds.attend(q, bt, lens, 1 / math.sqrt(dk), None).float().cpu().numpy()[0]
    assert_close(out, np.broadcast_to(ref, out.shape), f"mla huge context {kv}")
    lse = ds.lse.cpu().numpy()[0]
    assert np.allclose(lse, math.log(L), rtol=0, atol=1e-4), (lse.min(), lse.max(), math.log(L))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("jumps", [((128 + 5, 7.0),), ((128 + 2, 5.0), (128 + 5, 7.0)),
                                   ((128 + 1, 7.0), (128 + 6, 5.0)), ((160 + 12, 6.0),)],
                         ids=["one_token_upper_half", "halves_different_upper_higher",
                              "halves_different_lower_higher", "one_token_second_block"])
@pytest.mark.parametrize("head", [0, 45])
def test_mla_score_jump_single_tokens(kv, jumps, head):
    """Single tokens whose keys align with one head's query jump far above
    the first tile's scores. Token t of a 32-token block sits in one of two
    lane halves by bit 2 of t, so a jump in one half only (and jumps of
    different size in the two halves of one block) must still give every lane
    of the head the same reference max; a jump in a head other than the
    first of its wave (head 45: wave 1, lane 13) must still make the
    workgroup redo the segment."""
    from oracle import attention
    hq, dk, dv, P, L = 128, 576, 512, 64, 256
    rng = np.random.default_rng(19)
    q = torch.from_numpy(rng.standard_normal((1, hq, dk)).astype(np.float32)).to(torch.bfloat16)
    sign = np.sign(q[0, head].float().numpy())
    sign[sign == 0] = 1
    vals = rng.standard_normal((L, dk)).astype(np.float32) * 0.01
    for t, a in jumps:
        vals[t] = a * sign
    scale = np.float32(7.0 / 448.0)
    cache = pkv.allocate_cache(4, 1, P, dk, dv, kv, latent=True, device=dev)
    if kv == "fp8":
        codes = e4m3.encode((vals / scale).astype(np.float32))
        k_hat = e4m3.DECODE[codes] * np.float64(scale)
        cache.k_pool[:, 0] = torch.from_numpy(codes.reshape(4, P, dk)).to(dev)
        cache.k_scale.fill_(float(scale))
        cache.v_scale = cache.k_scale
    else:
        kb = torch.from_numpy(vals).to(torch.bfloat16)
        k_hat = kb.double().numpy()
        cache.k_pool[:, 0] = kb.view(4, P, dk).to(dev)
    bt = torch.arange(4, dtype=torch.int32, device=dev).view(1, 4)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    sm = 1 / math.sqrt(dk)
    ds = pkv.DecodeStep(cache, hq, 1, L, 256, verify=False)
    out = ds.attend(q.to(dev), bt, lens, sm, None).float().cpu().numpy()[0]
    ref, lse_ref = attention.attend(q[0].double().numpy(), k_hat[:, None, :], k_hat[:, None, :dv], sm)
    assert_close(out, ref, f"mla single-token jump {kv} {jumps}")
    assert np.allclose(ds.lse.cpu().numpy()[0], lse_ref, rtol=0, atol=1e-3)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_mla_query_magnitudes(kv):
    """Queries whose size differs per head (2^-24 .. 2^10 times N(0,1)),
    within a head (magnitudes spread over 2^-8 .. 2^2, random signs), an
    all-zero head, a head of bf16 subnormals and a head with one 32x dim:
    the e4m3 kernel splits q per head into two e4m3 parts scaled by the
    head's largest value, so every such shape must still match the oracle.
    Ragged: 300 tokens, the last page holds 44."""
    from oracle import attention
    hq, dk, dv, P, L = 128, 576, 512, 64, 300
    n_pages = -(-L // P)
    rng = np.random.default_rng(31)
    q = rng.standard_normal((hq, dk))
    q *= np.exp2(rng.integers(-24, 11, size=(hq, 1)))                  # per-head size
    q[5:40] *= np.exp2(rng.uniform(-8, 2, size=(35, dk)))               # spread inside a head
    q[0] = 0.0                                                          # all zero
    q[1] = rng.choice([-1.0, 0.0, 1.0], size=dk) * rng.integers(1, 128, size=dk) * 2.0**-133  # subnormal
    q[2] = rng.standard_normal(dk)
    q[2, 17] = 32.0 * np.abs(q[2]).max()                                # one large dim
    qb = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).view(1, hq, dk)
    vals = rng.standard_normal((n_pages * P, dk)).astype(np.float32)
    cache = pkv.allocate_cache(n_pages, 1, P, dk, dv, kv, latent=True, device=dev)
    if kv == "fp8":
        scale = np.float32(np.abs(vals).max() / 448.0)
        codes = e4m3.encode((vals / scale).astype(np.float32))
        k_hat = e4m3.DECODE[codes] * np.float64(scale)
        cache.k_pool[:, 0] = torch.from_numpy(codes.reshape(n_pages, P, dk)).to(dev)
        cache.k_scale.fill_(float(scale))
        cache.v_scale = cache.k_scale
    else:
        kb = torch.from_numpy(vals).to(torch.bfloat16)
        k_hat = kb.double().numpy()
        cache.k_pool[:, 0] = kb.view(n_pages, P, dk).to(dev)
    k_hat = k_hat[:L]
    bt = torch.arange(n_pages, dtype=torch.int32, device=dev).view(1, n_pages)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    sm = 1 / math.sqrt(dk)
    ds = pkv.DecodeStep(cache, hq, 1, L, 128, verify=False)
    out = ds.attend(qb.to(dev), bt, lens, sm, None).float().cpu().numpy()[0]
    ref, lse_ref = attention.attend(qb[0].double().numpy(), k_hat[:, None, :], k_hat[:, None, :dv], sm)
    assert_close(out, ref, f"mla query magnitudes {kv}")
    assert_lse_close(ds.lse.cpu().numpy()[0], lse_ref, f"mla query magnitudes {kv} lse")


def _gqa_direct_case(kv, vals_k, vals_v, bt_pages, L, hq, P, split, num_pages, seed=11):
    """Write K/V rows straight into a pool (token t of the request lives in
    page bt_pages[t // P]) and decode one request without the tag check."""
    from oracle import attention
    dk = vals_k.shape[1]
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((1, hq, dk)).astype(np.float32)).to(torch.bfloat16)
    cache = pkv.allocate_cache(num_pages, 1, P, dk, dk, kv, device=dev)
    k_hat = np.zeros_like(vals_k, dtype=np.float64)
    v_hat = np.zeros_like(vals_v, dtype=np.float64)
    if kv == "fp8":
        ks = np.float32(np.abs(vals_k).max() / 448.0)
        vs = np.float32(np.abs(vals_v).max() / 448.0)
        kc = e4m3.encode((vals_k / ks).astype(np.float32))
        vc = e4m3.encode((vals_v / vs).astype(np.float32))
        k_hat[:], v_hat[:] = e4m3.DECODE[kc] * np.float64(ks), e4m3.DECODE[vc] * np.float64(vs)
        cache.k_scale.fill_(float(ks))
        cache.v_scale.fill_(float(vs))
        kt, vt = torch.from_numpy(kc), torch.from_numpy(vc)
    else:
        kt = torch.from_numpy(vals_k).to(torch.bfloat16)
        vt = torch.from_numpy(vals_v).to(torch.bfloat16)
        k_hat[:], v_hat[:] = kt.double().numpy(), vt.double().numpy()
    keep = []
    for t in range(L):
        pg = bt_pages[t // P]
        if 0 <= pg < num_pages:
            cache.k_pool[pg, 0, t % P] = kt[t].to(dev)
            cache.v_pool[pg, 0, t % P] = vt[t].to(dev)
            keep.append(t)
    bt = torch.tensor([bt_pages], dtype=torch.int32, device=dev)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    sm = 1 / math.sqrt(dk)
    ds = pkv.DecodeStep(cache, hq, 1, L, split, verify=False)
    out = ds.attend(q.to(dev), bt, lens, sm, None).float().cpu().numpy()[0]
    keep = np.asarray(keep)
    ref, _ = attention.attend(q[0].double().numpy(), k_hat[keep][:, None, :], v_hat[keep][:, None, :], sm)
    return out, ref


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("jump_page", [1, 7, 15])
def test_gqa_score_jump_far_above_the_first_group(kv, jump_page):
    """Keys of a later page aligned with head 0's query put its score far
    above every score of the first 16-token group: the softmax reference must
    move (or the unit be recomputed) without losing accuracy."""
    hq, dk, P, L = 8, 128, 16, 256
    rng = np.random.default_rng(12)
    q_sign = np.sign(torch.from_numpy(np.random.default_rng(11).standard_normal((1, hq, dk))
                                      .astype(np.float32)).to(torch.bfloat16)[0, 0].float().numpy())
    q_sign[q_sign == 0] = 1
    vals_k = rng.standard_normal((L, dk)).astype(np.float32) * 0.01
    vals_k[P * jump_page:P * (jump_page + 1)] = 7.0 * q_sign
    vals_v = rng.standard_normal((L, dk)).astype(np.float32)
    out, ref = _gqa_direct_case(kv, vals_k, vals_v, list(range(16)), L, hq, P, 256, 16)
    assert_close(out, ref, f"gqa score jump {kv} page {jump_page}")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("bad", [[0], [3], [0, 1], [6]])
def test_gqa_out_of_pool_pages_left_out_without_tag_check(kv, bad):
    """With the no-op tracker a block-table entry outside the pool is never
    read and its tokens are left out, including the unit's first page."""
    hq, dk, P, L, n_pages = 8, 128, 16, 100, 8
    rng = np.random.default_rng(13)
    vals_k = rng.standard_normal((L, dk)).astype(np.float32)
    vals_v = rng.standard_normal((L, dk)).astype(np.float32)
    pages = [1, 2, 3, 4, 5, 6, 7]
    for j in bad:
        pages[j] = n_pages + 5 if j % 2 == 0 else -3
    out, ref = _gqa_direct_case(kv, vals_k, vals_v, pages, L, hq, P, 112, n_pages)
    assert_close(out, ref, f"gqa out-of-pool pages {bad} {kv}")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_batch_above_64(kv):
    """More requests than one wave has lanes (the e4m3 path's one-workgroup-
    per-unit launch), ragged lengths including one-token requests."""
    lens = [int(x) for x in np.random.default_rng(21).integers(1, 400, size=70)]
    lens[3] = 1
    lens[40] = 16
    w = W.custom("b70", 81, lens, hq=16, hkv=2, dk=128, dv=128, page=16, split=64)
    st = State(w, kv)
    _check_requests(st, range(0, w.batch, 3))
