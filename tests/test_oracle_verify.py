"""Pins of the oracle's integrity check: a hand-made worked example of the
rule in the pages, special cases, and a brute-force restatement over random
block tables."""
import json
import os

import numpy as np

import workloads as W
from oracle import verify

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "integrity_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    tags = np.array(g["page_tags"], dtype=np.uint32)
    for p in g["reallocate"]:
        tags[p] += 1
    got = verify.verify(tags, np.array(g["block_table"]), np.array(g["expected_tags"], dtype=np.uint32),
                        np.array(g["seq_lens"]), g["page_size"])
    assert got.tolist() == g["expected_abort"]


def test_no_reallocation_no_abort():
    w = W.sweep(8)
    assert verify.verify(w.page_tags, w.block_table, w.expected_tags, w.seq_lens, 16).sum() == 0


def test_tiny_flags_the_request_that_reads_the_bumped_page():
    w = W.tiny()
    got = verify.verify(w.page_tags, w.block_table, w.expected_tags, w.seq_lens, w.page_size)
    p = int(w.reallocated_pages[0])
    readers = [b for b in range(w.batch)
               if p in w.block_table[b, :-(-int(w.seq_lens[b]) // w.page_size)]]
    assert got.tolist() == [1 if b in readers else 0 for b in range(w.batch)]
    assert got.sum() == 1


def test_bump_of_an_unused_page_aborts_nothing():
    w = W.tiny(bump_unused=True)
    assert verify.verify(w.page_tags, w.block_table, w.expected_tags, w.seq_lens, w.page_size).sum() == 0


def test_shared_page_aborts_every_reader():
    tags = np.arange(8, dtype=np.uint32) * 7
    bt = np.array([[0, 3], [3, 1], [2, 4], [3, -1]])
    exp = tags[np.maximum(bt, 0)].copy()
    tags[3] += 1
    got = verify.verify(tags, bt, exp, np.array([5, 8, 8, 2]), 4)
    assert got.tolist() == [1, 1, 0, 1]


def test_entries_past_the_length_are_ignored():
    tags = np.array([1, 2, 3], dtype=np.uint32)
    bt = np.array([[0, 99, -5]])
    exp = np.array([[1, 0, 0]], dtype=np.uint32)
    assert verify.verify(tags, bt, exp, np.array([4]), 4).tolist() == [0]
    assert verify.verify(tags, bt, exp, np.array([5]), 4).tolist() == [1]


def test_random_against_set_formulation():
    rng = np.random.default_rng(11)
    for _ in range(50):
        n_pages = int(rng.integers(1, 40))
        B = int(rng.integers(1, 6))
        P = int(rng.choice([1, 4, 16]))
        maxp = int(rng.integers(1, 6))
        tags = rng.integers(0, 2**32, size=n_pages, dtype=np.uint64).astype(np.uint32)
        bt = rng.integers(-2, n_pages + 2, size=(B, maxp))
        exp = tags[np.clip(bt, 0, n_pages - 1)].copy()
        flip = rng.random((B, maxp)) < 0.1
        exp[flip] ^= 1
        lens = rng.integers(0, maxp * P + 1, size=B)
        got = verify.verify(tags, bt, exp, lens, P)
        for b in range(B):
            used = set(range(-(-int(lens[b]) // P)))
            bad = {j for j in used if not (0 <= bt[b, j] < n_pages) or tags[bt[b, j]] != exp[b, j]}
            assert got[b] == (1 if bad else 0)


def test_request_longer_than_its_row_is_aborted():
    """Reading of the section's rule: tokens beyond the block-table row have no
    page, like an id outside the pool, so the request is aborted."""
    tags = np.arange(8, dtype=np.uint32)
    bt = np.array([[0, 1], [2, 3]])
    exp = tags[bt]
    got = verify.verify(tags, bt, exp, np.array([8, 9]), 4)
    assert got.tolist() == [0, 1]
