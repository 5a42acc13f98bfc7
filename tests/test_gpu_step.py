"""GPU tests of the step in two launches (pkv_step_decode -> pkv_step_combine).

Its contract is the three-launch step (pkv_verify_append with each request's
new token at its last position -> pkv_decode_attn -> pkv_combine) bit for
bit: abort flags, outputs, lse and the cache contents afterwards. Before each
run the new token's row in the pool is overwritten with NaN codes, so a
decode that read the pool's row instead of the new token's values, or an
append that did not happen, shows at once. Full-size runs are also compared
with the float64 oracle ("Smaller, faster, safer", sections "Quantizing the
KV cache" and "Protecting a shared KV cache")."""
import math

import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import step as ostep
from tests.gpu_state import State
from tests.test_gpu_decode import _check_requests

pytestmark = pytest.mark.gpu
dev = "cuda"


class TwoLaunchState(State):
    """State whose step is the two-launch form."""

    def run(self, fused: bool = True):
        out = self.step.step2(self.q, self.block_table, self.expected, self.seq_lens,
                              self.w.sm_scale, self.new_k, self.new_v)
        torch.cuda.synchronize()
        return out


def _last_slots(st, lens):
    """The row of each request's last position (-1: no token, or a page
    outside the block table or the pool)."""
    P = st.w.page_size
    bt = st.block_table.cpu().numpy()
    out = np.full(len(lens), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        L = int(L)
        if L >= 1 and (L - 1) // P < bt.shape[1]:
            pid = int(bt[b, (L - 1) // P])
            if 0 <= pid < st.w.num_pages:
                out[b] = pid * P + (L - 1) % P
    return out


def _poison_rows(st, slots):
    """NaN codes (or bf16 NaN) in every kv head of the given pool rows."""
    P = st.w.page_size
    c = st.cache
    nan_k = 0x7F if st.kv_dtype == "fp8" else float("nan")
    for s in slots:
        if s < 0:
            continue
        page, row = int(s) // P, int(s) % P
        if st.kv_dtype == "fp8":
            c.k_pool[page, :, row, :] = nan_k
            if c.v_pool is not None:
                c.v_pool[page, :, row, :] = nan_k
        else:
            c.k_pool[page, :, row, :] = float("nan")
            if c.v_pool is not None:
                c.v_pool[page, :, row, :] = float("nan")


def _prepare(w, kv, split, max_seq_len=None, row_scales=False, edit=None, verify=True):
    """Two identical states (three-launch and two-launch), with the same
    device-side edits (lengths, block table, recorded tags) and the same
    poisoned last rows."""
    sts = []
    for _ in range(2):
        st = State(w, kv, split_tokens=split, row_scales=row_scales)
        if edit is not None:
            edit(st)
        msl = max_seq_len if max_seq_len is not None else max(1, int(st.seq_lens.max()))
        st.max_seq_len = msl
        st.step = pkv.DecodeStep(st.cache, w.num_q_heads, w.batch, msl, split, verify, dev)
        lens = st.seq_lens.cpu().numpy()
        st.last_slot = _last_slots(st, lens)
        _poison_rows(st, st.last_slot)
        torch.cuda.synchronize()
        sts.append(st)
    return sts


def _pool_bytes(t):
    return t.view(torch.uint8) if t.dtype == torch.uint8 else t.view(torch.int16)


def _run_both_and_compare(a, b):
    slot = torch.from_numpy(a.last_slot).to(dev)
    a.step.run(a.q, a.block_table, a.expected, a.seq_lens, a.w.sm_scale, a.new_k, a.new_v, slot)
    b.step.step2(b.q, b.block_table, b.expected, b.seq_lens, b.w.sm_scale, b.new_k, b.new_v)
    torch.cuda.synchronize()
    assert torch.equal(a.step.abort, b.step.abort), (a.step.abort, b.step.abort)
    assert torch.equal(a.step.out.view(torch.int16), b.step.out.view(torch.int16)), "out differs"
    assert torch.equal(a.step.lse.view(torch.int32), b.step.lse.view(torch.int32)), "lse differs"
    assert torch.equal(_pool_bytes(a.cache.k_pool), _pool_bytes(b.cache.k_pool)), "K pool differs"
    if a.cache.v_pool is not None:
        assert torch.equal(_pool_bytes(a.cache.v_pool), _pool_bytes(b.cache.v_pool)), \
            "V pool differs"
    if a.cache.k_row_scale is not None:
        assert torch.equal(a.cache.k_row_scale.view(torch.int32),
                           b.cache.k_row_scale.view(torch.int32))
        assert torch.equal(a.cache.v_row_scale.view(torch.int32),
                           b.cache.v_row_scale.view(torch.int32))
    return a.step.abort.cpu().numpy(), a.step.out.float().cpu().numpy()


# lengths around page, tile and split edges; requests 9 .. 11 are edited
LENS = [1, 15, 16, 17, 33, 250, 513, 1000, 64, 700, 400, 129]


def _edits(st):
    """Request 9: a recorded tag of its first page changed; 10: a block-table
    entry in its middle outside the pool; 11: the recorded tag of its last
    page (the one the new token goes to) changed; 8: empty (length 0)."""
    e = st.expected.view(torch.int32)
    e[9, 0] ^= 1
    st.block_table[10, 12] = st.w.num_pages + 7
    last = (int(st.seq_lens[11]) - 1) // st.w.page_size
    e[11, last] ^= 1
    st.seq_lens[8] = 0


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("heads", [(16, 4), (16, 1), (8, 8), (16, 8), (64, 8)],
                         ids=["G4", "G16", "G1", "G2", "G8"])
@pytest.mark.parametrize("split", [64, 16], ids=["direct_merge", "looped_merge"])
def test_two_launch_step_equals_three_launches(kv, heads, split):
    hq, hkv = heads
    w = W.custom(f"step_{hq}_{hkv}", 3100 + hq + hkv, LENS, hq=hq, hkv=hkv, dk=128, dv=128,
                 page=16, per_head=True, n_realloc=2)
    a, b = _prepare(w, kv, split, edit=_edits)
    flags, out = _run_both_and_compare(a, b)
    want = ostep.flags(w).astype(np.uint8)
    want[8], want[9], want[10], want[11] = 0, 1, 1, 1
    assert np.array_equal(flags, want), (flags, want)
    assert np.all(out[8] == 0.0)
    ok = [i for i in range(w.batch) if not flags[i] and i != 8]
    assert ok and np.all(np.isfinite(out[ok])), "a standing request has non-finite output"


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_two_launch_step_page32(kv):
    """Page 32, 128-token splits (four pages a split), the same edits."""
    w = W.custom("step_p32", 3170, LENS, hq=64, hkv=8, dk=128, dv=128, page=32, per_head=True,
                 n_realloc=2)

    def edit(st):
        e = st.expected.view(torch.int32)
        e[9, 0] ^= 1
        st.block_table[10, 6] = st.w.num_pages + 7
        e[11, (int(st.seq_lens[11]) - 1) // 32] ^= 1
        st.seq_lens[8] = 0

    a, b = _prepare(w, kv, 128, edit=edit)
    assert pkv.pkv_step_launches(b.cache, 64, 128) == 2
    flags, out = _run_both_and_compare(a, b)
    want = ostep.flags(w).astype(np.uint8)
    want[8], want[9], want[10], want[11] = 0, 1, 1, 1
    assert np.array_equal(flags, want), (flags, want)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_two_launch_step_without_the_check(kv):
    """No recorded tags: no request is aborted (the tag edits change
    nothing), a page outside the pool is still never read, and the result is
    the append (no check) -> decode -> merge one, bit for bit."""
    w = W.custom("step_nocheck", 3150, LENS, hq=16, hkv=4, dk=128, dv=128, page=16,
                 per_head=True, n_realloc=2)
    a, b = _prepare(w, kv, 64, edit=_edits, verify=False)
    flags, out = _run_both_and_compare(a, b)
    assert not flags.any()
    ok = [i for i in range(w.batch) if i not in (8, 10)]
    assert np.all(np.isfinite(out[ok]))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_two_launch_step_page64_and_overlong_requests(kv):
    """Page 64, 128-token splits; max_seq_len 600 leaves requests 7 (1000,
    standing: NaN output, new token appended) and 9 (700, aborted: zeros)
    without units, so the merge checks them in full."""
    w = W.custom("step_p64", 3200, LENS, hq=16, hkv=2, dk=128, dv=128, page=64, per_head=True)

    def edit(st):
        st.expected.view(torch.int32)[9, 3] ^= 1
        st.seq_lens[1] = -3

    a, b = _prepare(w, kv, 128, max_seq_len=600, edit=edit)
    flags, out = _run_both_and_compare(a, b)
    assert flags[7] == 0 and flags[9] == 1 and flags[1] == 0
    assert np.all(np.isnan(out[7])) and np.all(out[9] == 0.0) and np.all(out[1] == 0.0)
    # the over-long standing request's token was still appended
    s = int(a.last_slot[7])
    row = b.cache.k_pool[s // 64, :, s % 64, :]
    poisoned = (row == 0x7F) if kv == "fp8" else torch.isnan(row)
    assert s >= 0 and not poisoned.any()


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("case", ["L1", "L15", "L700", "tag", "empty", "overlong", "outside_pool"])
def test_one_request(kv, case):
    """One request (its units' places need no lookup, so their loads go out
    beside its length): the two-launch step equals the three-launch one bit
    for bit, through tiny, aborted, empty and over-long requests, and a
    standing request matches the oracle."""
    L = {"L1": 1, "L15": 15}.get(case, 700)
    w = W.custom(f"one_{case}", 3500 + L, [L], hq=16, hkv=4, dk=128, dv=128, page=16,
                 per_head=True)

    def edit(st):
        if case == "tag":
            st.expected.view(torch.int32)[0, 20] ^= 1
        elif case == "empty":
            st.seq_lens[0] = 0
        elif case == "outside_pool":
            st.block_table[0, 3] = st.w.num_pages + 1

    msl = 600 if case == "overlong" else None
    a, b = _prepare(w, kv, 64, max_seq_len=msl, edit=edit)
    flags, out = _run_both_and_compare(a, b)
    assert flags[0] == (1 if case in ("tag", "outside_pool") else 0)
    if case in ("tag", "outside_pool", "empty"):
        assert np.all(out[0] == 0.0)
    elif case == "overlong":
        assert np.all(np.isnan(out[0]))
    else:
        _check_requests(TwoLaunchStateFrom(b), [0])


def TwoLaunchStateFrom(st):
    """The same device state, its step run as the two-launch form again (the
    pool already holds the appended row; appending it again changes nothing)."""
    st.__class__ = TwoLaunchState
    return st


@pytest.mark.parametrize("case", ["row_scales", "head_dim_64", "long_split", "latent"])
def test_three_launch_fallback_shapes(case):
    """Shapes without the two-launch form run the three launches inside the
    same two calls (the check and append with the slot taken from the
    length): still the three-launch results bit for bit."""
    kv, split, rows, msl = "fp8", 64, False, None
    if case == "row_scales":
        w = W.custom("fb_rows", 3300, LENS, hq=16, hkv=4, dk=128, dv=128, page=16, n_realloc=2)
        rows = True
    elif case == "head_dim_64":
        w = W.custom("fb_d64", 3301, LENS, hq=8, hkv=2, dk=64, dv=64, page=16, n_realloc=2)
    elif case == "long_split":
        # 4096-token splits at page 16: 256 pages per unit, past the step form's 128
        w = W.custom("fb_long", 3302, [5000, 4097, 300, 9000], hq=16, hkv=4, dk=128, dv=128,
                     page=16, per_head=True, n_realloc=2)
        split = 4096
    else:
        w = W.custom("fb_latent", 3303, [1, 64, 65, 700, 1500], hq=16, hkv=1, dk=576, dv=512,
                     page=64, latent=True, n_realloc=1)
        split = 256

    def edit(st):
        st.expected.view(torch.int32)[1, 0] ^= 1

    a, b = _prepare(w, kv, split, max_seq_len=msl, row_scales=rows, edit=edit)
    flags, out = _run_both_and_compare(a, b)
    want = ostep.flags(w).astype(np.uint8)
    want[1] = 1
    assert np.array_equal(flags, want), (flags, want)
    ok = np.flatnonzero(want == 0)
    assert ok.size and np.all(np.isfinite(out[ok]))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_no_check_append_stays_inside_the_pool_and_the_row(kv):
    """Without the check a request may still reach the step with a length
    past its block-table row, or with the page of its last position outside
    the pool. Neither launch form may append then (no read past the row, no
    write past the pool); both give the same flags, outputs and pools."""
    w = W.custom("step_bounds", 3160, [300, 450, 200, 100], hq=16, hkv=4, dk=128, dv=128,
                 page=16, per_head=True)

    def edit(st):
        P, mp = st.w.page_size, st.block_table.shape[1]
        st.block_table[1, (450 - 1) // P] = st.w.num_pages + 3  # last page outside the pool
        st.seq_lens[3] = mp * P + 5                             # past the last request's row

    a, b = _prepare(w, kv, 64, max_seq_len=450, edit=edit, verify=False)
    before = _pool_bytes(b.cache.k_pool).clone()
    flags, out = _run_both_and_compare(a, b)
    assert not flags.any()
    assert np.all(np.isnan(out[3]))
    # only requests 0 and 2 appended: every other row is as before
    after = _pool_bytes(b.cache.k_pool)
    changed = torch.nonzero((after != before).reshape(after.shape[0], after.shape[1],
                                                      after.shape[2], -1).any(-1).any(1))
    rows = {int(p) * w.page_size + int(r) for p, r in changed.tolist()}
    assert rows <= {int(a.last_slot[0]), int(a.last_slot[2])}, rows


def test_sweep_b64_full_size_sampled_against_oracle():
    """The measured workload through the two-launch step, sampled requests
    against the float64 oracle (the new token's row comes from its values)."""
    st = TwoLaunchState(W.sweep(64), "fp8")
    _poison_rows(st, _last_slots(st, st.seq_lens.cpu().numpy()))
    _check_requests(st, [0, 31, 63], kv_heads=[3])
    # the appended rows are in the pool afterwards: the three-launch decode
    # of the same requests, with nothing appended, gives the same bits
    out2 = st.step.out.clone()
    lse2 = st.step.lse.clone()
    st.step.attend(st.q, st.block_table, st.seq_lens, st.w.sm_scale, st.step.abort)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), st.step.out.view(torch.int16))
    assert torch.equal(lse2.view(torch.int32), st.step.lse.view(torch.int32))


def test_long_context_full_size_sampled_against_oracle():
    """The long-context workload (4 x 131,072 tokens, page 64, 256-token
    chunks) as bench.py times it, through the two-launch step: two requests
    against the float64 oracle (all 512 chunks of each merged), their new
    tokens' rows poisoned in the pool beforehand."""
    st = TwoLaunchState(W.long_context(), "fp8")
    assert pkv.pkv_step_launches(st.cache, st.w.num_q_heads, st.step.split_tokens) == 2
    _poison_rows(st, _last_slots(st, st.seq_lens.cpu().numpy()))
    _check_requests(st, [0, 3], kv_heads=[5])


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("make", [lambda: W.sweep(64), W.long_context],
                         ids=["sweep_b64", "long_b4"])
def test_zero_query_sentinel_two_launch(make, kv):
    """q = 0: every weight is 1 / L_b, so lse = ln L_b to 1e-5 for every
    (request, head), which a tile lost or read twice, or a missing new row,
    would move."""
    w = make()
    st = TwoLaunchState(w, kv)
    _poison_rows(st, _last_slots(st, st.seq_lens.cpu().numpy()))
    st.q.zero_()
    st.run()
    lse = st.step.lse.cpu().numpy().astype(np.float64)
    flags = ostep.flags(w)
    assert np.array_equal(st.step.abort.cpu().numpy(), flags)
    for b in range(w.batch):
        if flags[b]:
            assert np.all(np.isneginf(lse[b]))
        else:
            err = np.abs(lse[b] - math.log(int(w.seq_lens[b])))
            assert err.max() <= 1e-5, f"{w.name} request {b}: lse off ln L by {err.max():.2e}"


def test_two_launch_graph_replays_match_eager():
    """The two launches captured as a HIP graph and replayed (eager work and
    synchronisations between replays) give the eager step's bits each time."""
    w = W.custom("step_graph", 3400, LENS, hq=16, hkv=4, dk=128, dv=128, page=16,
                 per_head=True, n_realloc=2)
    st = TwoLaunchState(w, "fp8", split_tokens=64)
    st.run()
    ref_out = st.step.out.clone()
    ref_lse = st.step.lse.clone()
    ref_abort = st.step.abort.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step.step2(st.q, st.block_table, st.expected, st.seq_lens, w.sm_scale, st.new_k,
                      st.new_v)
    for i in range(3):
        st.step.out.zero_()
        st.step.lse.zero_()
        st.step.abort.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.step.out.view(torch.int16), ref_out.view(torch.int16)), i
        assert torch.equal(st.step.lse.view(torch.int32), ref_lse.view(torch.int32)), i
        assert torch.equal(st.step.abort, ref_abort), i
