"""Pins for the oracle's router and pair permutation (CPU only).

Brute force in plain Python on small inputs (including forced ties),
library softmax, and the invariants the routing must satisfy.
"""

import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("T,E,k", [(5, 8, 2), (17, 16, 4), (3, 128, 8), (4, 6, 6)])
def test_topk_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    lg = rng.standard_normal((T, E), dtype=np.float32)
    ids, w = oracle.route_topk(lg, k)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(lg[t], k)


def test_topk_ties_go_to_lower_id():
    lg = np.array([[0.5, 1.0, 1.0, 0.5, 1.0, -2.0],
                   [0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
                   [-0.0, 0.0, -1.0, 3.0, 3.0, -0.0]], dtype=np.float32)
    ids, w = oracle.route_topk(lg, 4)
    assert ids.tolist() == [[1, 2, 4, 0], [0, 1, 2, 3], [3, 4, 0, 1]]
    # equal logits get equal weights
    assert w[1, 0] == w[1, 3] == pytest.approx(0.25, abs=1e-15)


def test_weights_are_softmax_over_the_selection():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((64, 32), dtype=np.float32) * 3
    ids, w = oracle.route_topk(lg, 8)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0), "weights follow the logit order"
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8


def test_k_equals_e_is_the_full_softmax():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((7, 10), dtype=np.float32)
    ids, w = oracle.route_topk(lg, 10)
    full = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-14)


def test_no_renormalisation_keeps_full_softmax_probabilities():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((9, 12), dtype=np.float32)
    ids, w = oracle.route_topk(lg, 3, renormalize=False)
    full = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-14)
    assert np.all(w.sum(1) < 1.0)


def test_large_logits_do_not_overflow():
    lg = np.array([[1000.0, 999.0, -1000.0, 0.0]], dtype=np.float32)
    ids, w = oracle.route_topk(lg, 2)
    assert ids.tolist() == [[0, 1]]
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-14)


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (9, 8, 2), (33, 16, 4), (50, 128, 8)])
def test_permutation_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    lg = rng.standard_normal((T, E), dtype=np.float32)
    ids, _ = oracle.route_topk(lg, k)
    sp, pos, off = oracle.permute_pairs(ids, E)
    flat = ids.reshape(-1).tolist()
    P = T * k
    want = sorted(range(P), key=lambda p: (flat[p], p))
    assert sp.tolist() == want
    assert sorted(sp.tolist()) == list(range(P))
    for p in range(P):
        assert sp[pos[p]] == p
    counts = [flat.count(e) for e in range(E)]
    assert off[0] == 0 and off[E] == P
    assert [int(off[e + 1] - off[e]) for e in range(E)] == counts
    for e in range(E):
        for i in range(off[e], off[e + 1]):
            assert flat[sp[i]] == e


def test_permutation_with_empty_experts():
    ids = np.array([[3, 1], [3, 1], [1, 3]], dtype=np.int32)
    sp, pos, off = oracle.permute_pairs(ids, 5)
    assert off.tolist() == [0, 0, 3, 3, 6, 6]
    assert sp.tolist() == [1, 3, 4, 0, 2, 5]
