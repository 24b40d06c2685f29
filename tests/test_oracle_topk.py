"""Pins of the oracle's top-k against definitions that do not share its code.

The oracle takes the first k entries of a stable descending sort. Here the
selection is checked against the rank definition written out as loops
(rank(s) = #{j: S_j > S_s} + #{j < s: S_j == S_s}), against closed forms,
and on tie-heavy inputs where a wrong tie rule or a sign slip would show.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_topk(scores, k):
    """Rank definition with Python loops (tiny inputs only)."""
    s = [float(x) for x in scores]
    n = len(s)
    k_eff = min(k, n)
    out = [-1] * k
    for i in range(n):
        rank = 0
        for j in range(n):
            if s[j] > s[i] or (s[j] == s[i] and j < i):
                rank += 1
        if rank < k_eff:
            out[rank] = i
    return out


def brute_topk_np(scores, k):
    """Same rank definition, vectorised (O(n^2) memory; n up to a few thousand)."""
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    idx = np.arange(n)
    gt = (s[None, :] > s[:, None]).sum(axis=1)
    eq_before = ((s[None, :] == s[:, None]) & (idx[None, :] < idx[:, None])).sum(axis=1)
    rank = gt + eq_before
    out = np.full(k, -1, np.int32)
    keep = rank < min(k, n)
    out[rank[keep]] = idx[keep]
    return out


def test_golden_hand_case():
    g = json.load(open(os.path.join(GOLDEN, "indexer_hand.json")))
    s = np.asarray(g["scores"], np.float32)
    for k, want in g["topk"].items():
        assert O.topk_row(s, int(k)).tolist() == want


@settings(max_examples=300, deadline=None)
@given(st.lists(st.sampled_from([-2.0, -0.5, -0.0, 0.0, 0.25, 1.0, 3.0]), min_size=1, max_size=40),
       st.integers(1, 48))
def test_rank_definition_with_ties(vals, k):
    s = np.asarray(vals, np.float32)
    assert O.topk_row(s, k).tolist() == brute_topk(s, k)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(-1e6, 1e6, allow_nan=False, width=32), min_size=1, max_size=60),
       st.integers(1, 64))
def test_rank_definition_continuous(vals, k):
    s = np.asarray(vals, np.float32)
    assert O.topk_row(s, k).tolist() == brute_topk(s, k)


def test_all_equal_is_index_order():
    for n, k in [(10, 4), (10, 10), (5, 9), (3000, 2048)]:
        got = O.topk_row(np.full(n, 7.5, np.float32), k)
        k_eff = min(n, k)
        assert got[:k_eff].tolist() == list(range(k_eff))
        assert (got[k_eff:] == -1).all()


def test_strictly_increasing_gives_latest_first():
    n, k = 5000, 2048
    got = O.topk_row(np.arange(n, dtype=np.float32), k)
    assert got.tolist() == list(range(n - 1, n - 1 - k, -1))


def test_k1_is_argmax_lowest_index():
    s = np.array([1.0, 5.0, 2.0, 5.0, 5.0], np.float32)
    assert O.topk_row(s, 1).tolist() == [1]


def test_signed_zero_ties():
    s = np.array([0.0, -0.0, 0.0, -0.0, -1.0, 1.0], np.float32)
    assert O.topk_row(s, 6).tolist() == [5, 0, 1, 2, 3, 4]
    assert O.topk_row(s, 3).tolist() == [5, 0, 1]


def test_large_tie_classes_straddle_threshold():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 8, size=4000).astype(np.float32) / 8.0
    got = O.topk_row(s, 2048)
    assert np.array_equal(got, brute_topk_np(s, 2048))
    # within the straddling class the lowest indices are the ones kept
    thr = s[got[-1]]
    kept = np.sort(got[s[got] == thr])
    all_eq = np.flatnonzero(s == thr)
    assert np.array_equal(kept, all_eq[:kept.size])


def test_padding_and_uniqueness():
    rng = np.random.default_rng(0)
    for n in [1, 2, 63, 64, 65, 700]:
        s = rng.standard_normal(n).astype(np.float32)
        got = O.topk_row(s, 64)
        k_eff = min(n, 64)
        assert len(set(got[:k_eff].tolist())) == k_eff
        assert (got[:k_eff] >= 0).all() and (got[:k_eff] < n).all()
        assert (got[k_eff:] == -1).all()
        assert np.array_equal(got, brute_topk_np(s, 64))
