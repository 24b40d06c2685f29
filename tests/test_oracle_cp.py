"""Pins of the oracle's context-parallel merges.

Top-k merge: merging the shards' local top-k lists equals the top-k of the
whole row (a property of a total order, checked by brute force on rows with
ties, signed zeros, short rows and shards past the causal bound). Output
merge: the log-sum-exp merge of attentions over a partition of the selected
keys equals the attention over all of them (softmax over a union), and two
closed forms.
"""
import numpy as np
import pytest

from oracle import dsa_oracle as O
from test_oracle_topk import brute_topk_np


def _shards(n, P):
    edges = np.linspace(0, n, P + 1).astype(int)
    return list(zip(edges[:-1], edges[1:]))


def _local_pairs(scores, lo, hi, t, k):
    """Shard [lo, hi)'s local top-k of a query at position t: (scores, global keys)."""
    top = min(hi, t + 1)
    ps = np.full(k, -np.inf, np.float32)
    pi = np.full(k, -1, np.int32)
    if top > lo:
        loc = brute_topk_np(scores[lo:top], k)
        v = loc >= 0
        pi[v] = loc[v] + lo
        ps[v] = scores[lo:top][loc[v]]
    return ps, pi


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros"])
@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_merge_of_local_topk_is_global_topk(kind, P):
    rng = np.random.default_rng(P * 10 + len(kind))
    n, k = 3000, 256
    if kind == "normal":
        s = rng.standard_normal(n).astype(np.float32)
    elif kind == "ties":
        s = (rng.integers(0, 6, n) / 4.0).astype(np.float32)
    else:
        s = np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    for t in (n - 1, 1700, 100, 5):       # causal bound inside, before and past the shards
        pairs = [_local_pairs(s, lo, hi, t, k) for lo, hi in _shards(n, P)]
        ps = np.stack([p[0] for p in pairs])
        pi = np.stack([p[1] for p in pairs])
        assert np.array_equal(O.topk_merge(ps, pi, k), brute_topk_np(s[:t + 1], k)), (kind, P, t)


def test_merge_closed_forms():
    # equal scores across shards: the lower keys win, in key order
    ps = np.full((3, 4), 1.5, np.float32)
    pi = np.array([[0, 1, 2, 3], [10, 11, 12, 13], [20, 21, 22, 23]], np.int32)
    assert O.topk_merge(ps, pi, 6).tolist() == [0, 1, 2, 3, 10, 11]
    # empty entries never win; fewer candidates than k pad with -1
    pi2 = pi.copy()
    pi2[:, 2:] = -1
    assert O.topk_merge(ps, pi2, 8).tolist() == [0, 1, 10, 11, 20, 21, -1, -1]


def test_attention_merge_equals_whole_attention():
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((300, 576)) * 0.1
    q = rng.standard_normal((6, 576)) * 3.0
    whole_o, whole_l = O.sparse_mla_row(q, rows, 1 / np.sqrt(192))
    for P in (1, 2, 5):
        part = rng.integers(0, P, 300)
        parts = [O.sparse_mla_row(q, rows[part == p], 1 / np.sqrt(192)) for p in range(P)]
        o, l = O.attn_merge(np.stack([x[0] for x in parts]), np.stack([x[1] for x in parts]))
        np.testing.assert_allclose(o, whole_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l, whole_l, rtol=1e-13)


def test_attention_merge_closed_forms():
    o = np.stack([np.full((2, 512), 1.0), np.full((2, 512), 3.0)])
    l = np.array([[0.25, np.log(3.0)], [0.25, 0.0]])
    out, lse = O.attn_merge(o, l)
    np.testing.assert_allclose(out[0], 2.0)                 # equal LSEs: the mean
    np.testing.assert_allclose(out[1], (3 * 1.0 + 1 * 3.0) / 4)
    np.testing.assert_allclose(lse, [0.25 + np.log(2.0), np.log(4.0)])
    out2, lse2 = O.attn_merge(o, np.array([[-np.inf, 1.0], [-np.inf, -np.inf]]))
    assert (out2[0] == 0).all() and np.isneginf(lse2[0])  # no key anywhere
    np.testing.assert_allclose(out2[1], 1.0)              # one part: itself
    np.testing.assert_allclose(lse2[1], 1.0)
