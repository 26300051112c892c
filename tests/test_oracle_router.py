"""Pins for routing (oracle/router.py): exhaustive rank counts, brute force, library softmax."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle import topk_order, route, router_logits


def _rank_count_selected(z, k):
    """e is selected iff fewer than k experts precede it in the total order."""
    E = len(z)
    sel = set()
    for e in range(E):
        ahead = sum(1 for f in range(E) if (z[f] > z[e]) or (z[f] == z[e] and f < e))
        if ahead < k:
            sel.add(e)
    return sel


def test_topk_matches_rank_count_and_bruteforce():
    rng = np.random.default_rng(0)
    for trial in range(300):
        E = int(rng.integers(2, 10))
        k = int(rng.integers(1, E + 1))
        # integer-valued logits make ties frequent
        z = rng.integers(-3, 4, size=E).astype(np.float32)
        if trial % 3 == 0:
            z = rng.standard_normal(E).astype(np.float32)
        idx = topk_order(z, k)
        assert set(idx.tolist()) == _rank_count_selected(z, k)
        # brute force: best k-subset by (descending sorted values, then ascending indices)
        best = max(itertools.combinations(range(E), k),
                   key=lambda c: (sorted((float(z[e]) for e in c), reverse=True), [-e for e in sorted(c)]))
        assert set(idx.tolist()) == set(best)
        # rank order: non-increasing logits, ties by ascending index
        for a, b in zip(idx[:-1], idx[1:]):
            assert z[a] > z[b] or (z[a] == z[b] and a < b)


def test_ties_and_signed_zero():
    z = np.array([1.0, 2.0, 2.0, -0.0, 0.0, 2.0], np.float32)
    assert topk_order(z, 3).tolist() == [1, 2, 5]
    assert topk_order(z, 5).tolist() == [1, 2, 5, 0, 3]
    with pytest.raises(ValueError):
        topk_order(np.array([0.0, np.nan], np.float32), 1)


def test_gates_match_library_softmax_and_renorm():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 16)).astype(np.float32)
    idx, w = route(z, 4, renorm=0)
    p = softmax(z.astype(np.float64), axis=1)
    for t in range(5):
        np.testing.assert_allclose(w[t], p[t, idx[t]], rtol=1e-6)
    idx2, w2 = route(z, 4, renorm=1)
    assert np.array_equal(idx, idx2)
    np.testing.assert_allclose(w2.sum(1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(w2, softmax(np.take_along_axis(z, idx, 1).astype(np.float64), axis=1), rtol=1e-6)
    idx3, w3 = route(z, 16)
    assert sorted(idx3[0].tolist()) == list(range(16))
    np.testing.assert_allclose(w3.sum(1), 1.0, rtol=1e-6)


def test_logits_against_exact_rationals():
    from fractions import Fraction
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 12)).astype(np.float32).astype(np.float64)
    wr = rng.standard_normal((5, 12)).astype(np.float32)
    bias = rng.standard_normal(5).astype(np.float32)
    z = router_logits(x, wr, bias)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(wr[e, h])) for h in range(12)) + Fraction(float(bias[e]))
            assert abs(float(z[t, e]) - float(exact)) <= 2 ** -23 * max(1.0, abs(float(exact)))
