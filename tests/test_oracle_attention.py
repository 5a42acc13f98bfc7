"""Pins of the oracle's attention and combine: pure-Python brute force,
torch's scaled_dot_product_attention (float64, CPU), scipy's logsumexp,
closed-form special cases, paged = contiguous, and split invariance."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention, combine


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _brute(q, k, v, sm):
    """Pure Python: fsum and math.exp, no NumPy reductions."""
    hq, hkv = q.shape[0], k.shape[1]
    g = hq // hkv
    outs, lses = [], []
    for h in range(hq):
        s = [sm * math.fsum(q[h, d] * k[t, h // g, d] for d in range(q.shape[1])) for t in range(k.shape[0])]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        outs.append([math.fsum(e[t] * v[t, h // g, d] for t in range(len(e))) / den
                     for d in range(v.shape[2])])
        lses.append(m + math.log(den))
    return np.array(outs), np.array(lses)


def test_brute_force_tiny_shapes():
    rng = np.random.default_rng(0)
    for L, hq, hkv, d in [(37, 4, 1, 16), (5, 2, 2, 8), (1, 3, 1, 4), (20, 8, 2, 12)]:
        q, k, v = _rand(rng, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d + 3)
        o, lse = attention.attend(q, k, v, 0.3)
        ob, lb = _brute(q, k, v, 0.3)
        assert np.allclose(o, ob, rtol=0, atol=1e-12)
        assert np.allclose(lse, lb, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(1)
    L, hq, hkv, d = 300, 16, 4, 32
    q, k, v = _rand(rng, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    sm = 1 / math.sqrt(d)
    o, _ = attention.attend(q, k, v, sm)
    g = hq // hkv
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    qt = torch.from_numpy(q)[:, None, :].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm)[:, 0, :].numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)


def test_lse_matches_scipy():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 50, 1, 8), _rand(rng, 50, 1, 8)
    _, lse = attention.attend(q, k, v, 0.7)
    for h in range(4):
        assert abs(lse[h] - logsumexp(0.7 * (k[:, 0, :] @ q[h]))) < 1e-12


def test_weights_sum_to_one_and_match_output():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 123, 2, 16), _rand(rng, 123, 2, 16)
    w = attention.weights(q, k, 0.25)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    o, _ = attention.attend(q, k, v, 0.25)
    for h in range(8):
        assert np.allclose(o[h], w[h] @ v[:, h // 4, :], atol=1e-12)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 1, 1, 8), _rand(rng, 1, 1, 5)
    o, lse = attention.attend(q, k, v, 0.5)
    assert np.allclose(o, np.repeat(v[0], 4, axis=0), atol=0)
    assert np.allclose(lse, 0.5 * (q @ k[0, 0]), atol=1e-14)


def test_equal_keys_or_zero_query_give_the_mean_value():
    rng = np.random.default_rng(5)
    k = np.repeat(_rand(rng, 1, 1, 8), 40, axis=0)
    v = _rand(rng, 40, 1, 6)
    o, lse = attention.attend(_rand(rng, 2, 8), k, v, 1.0)
    assert np.allclose(o, v[:, 0, :].mean(axis=0)[None], atol=1e-13)
    o2, lse2 = attention.attend(np.zeros((2, 8)), _rand(rng, 40, 1, 8), v, 1.0)
    assert np.allclose(o2, v[:, 0, :].mean(axis=0)[None], atol=1e-13)
    assert np.allclose(lse2, math.log(40), atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 30, 2, 16), _rand(rng, 30, 2, 16)
    o, lse = attention.attend(q, k, v, 0.2)
    o2, lse2 = attention.attend(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.2)
    assert np.allclose(o, o2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)


def test_paged_gather_equals_contiguous():
    rng = np.random.default_rng(7)
    P, hkv, d, L = 16, 2, 8, 70
    n_pages = 12
    contig = _rand(rng, L, hkv, d)
    perm = rng.permutation(n_pages)
    pool = np.full((n_pages, hkv, P, d), np.nan)
    for t in range(L):
        pool[perm[t // P], :, t % P, :] = contig[t]
    got = attention.gather(pool, perm, L, P)
    assert np.array_equal(got, contig)


@pytest.mark.parametrize("S", [1, 16, 64, 100, 1000])
def test_split_then_combine_equals_unsplit(S):
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 257, 2, 16), _rand(rng, 257, 2, 12)
    o, lse = attention.attend(q, k, v, 0.4)
    po, pl = combine.split_partials(q, k, v, 0.4, S)
    assert po.shape[0] == combine.num_splits(257, S)
    oc, lc = combine.combine(po, pl)
    assert np.allclose(oc, o, atol=1e-12) and np.allclose(lc, lse, atol=1e-12)


def test_combine_of_one_split_is_identity():
    rng = np.random.default_rng(9)
    po, pl = _rand(rng, 1, 4, 6), _rand(rng, 1, 4)
    o, l = combine.combine(po, pl)
    assert np.array_equal(o, po[0]) and np.allclose(l, pl[0], atol=0)


def test_planted_sign_error_is_caught():
    """A mistaken sign inside the exponent would break the brute-force pin."""
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 2, 8), _rand(rng, 9, 1, 8), _rand(rng, 9, 1, 8)
    o, _ = attention.attend(-q, k, v, 0.5)  # mutant: negated scores
    ob, _ = _brute(q, k, v, 0.5)
    assert not np.allclose(o, ob, atol=1e-6)


# ------------------------------------------------- drafts verified together
def _masked_brute(q, k, v, sm):
    """The same quantity written as one masked softmax per (query, head):
    scores of tokens after the query's own position are -inf; math.fsum and
    math.exp only."""
    import math
    T, hq, _ = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    o = np.zeros((T, hq, v.shape[2]))
    for j in range(T):
        for h in range(hq):
            s = []
            for t in range(L):
                if t > L - T + j:
                    s.append(-math.inf)
                else:
                    s.append(sm * math.fsum(q[j, h, d] * k[t, h // g, d] for d in range(k.shape[2])))
            m = max(s)
            e = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
            den = math.fsum(e)
            for d in range(v.shape[2]):
                o[j, h, d] = math.fsum(e[t] * v[t, h // g, d] for t in range(L)) / den
    return o


def test_drafts_match_masked_brute_force():
    rng = np.random.default_rng(31)
    T, L, hq, hkv, D = 3, 9, 4, 2, 5
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((L, hkv, D))
    v = rng.standard_normal((L, hkv, D))
    o, lse = attention.attend_drafts(q, k, v, 0.7)
    assert np.allclose(o, _masked_brute(q, k, v, 0.7), rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_drafts_single_query_is_plain_decode_and_rows_are_prefix_decodes():
    rng = np.random.default_rng(32)
    L, hq, hkv, D = 12, 4, 1, 6
    q = rng.standard_normal((4, hq, D))
    k = rng.standard_normal((L, hkv, D))
    v = rng.standard_normal((L, hkv, D))
    o1, l1 = attention.attend_drafts(q[:1], k, v, 0.3)
    o, l = attention.attend(q[0], k, v, 0.3)
    assert np.array_equal(o1[0], o) and np.array_equal(l1[0], l)
    # the first of 4 drafts sees 9 tokens, the last all 12
    o4, _ = attention.attend_drafts(q, k, v, 0.3)
    assert np.allclose(o4[0], attention.attend(q[0], k[:9], v[:9], 0.3)[0], atol=1e-12)
    assert np.allclose(o4[3], attention.attend(q[3], k, v, 0.3)[0], atol=1e-12)


def test_drafts_edge_cases():
    rng = np.random.default_rng(33)
    D = 4
    v = rng.standard_normal((3, 1, D))
    k = rng.standard_normal((3, 1, D))
    q = rng.standard_normal((3, 2, D))
    # L == T: the first query sees only token 0, so its output is v_0 exactly
    o, lse = attention.attend_drafts(q, k, v, 1.0)
    assert np.allclose(o[0, :, :], v[0, 0][None, :], atol=1e-15)
    # L < T: the first queries see nothing
    o, lse = attention.attend_drafts(q, k[:2], v[:2], 1.0)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.allclose(o[1], v[0, 0][None, :], atol=1e-15)
