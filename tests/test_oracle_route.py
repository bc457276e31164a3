"""Pins for the oracle's routing (softmax, top-k, renormalised gates).

Each check compares the oracle with something other than itself: a
pure-Python selection loop, scipy's softmax, closed-form special cases.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import moe_oracle as O


def brute_topk(row, k):
    """Repeated arg-max by a left-to-right scan; a strictly larger value is
    needed to replace the current best, so equal values keep the lower index."""
    chosen = []
    for _ in range(k):
        best = None
        for i, v in enumerate(row):
            if i in chosen:
                continue
            if best is None or v > row[best]:
                best = i
        chosen.append(best)
    return chosen


@pytest.mark.parametrize("E,k", [(8, 4), (5, 2), (16, 1), (6, 6), (128, 4)])
def test_topk_matches_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 31 + k)
    # Draw from a small set of values so that ties are common.
    logits = rng.integers(-3, 4, size=(64, E)).astype(np.float64) * 0.25
    idx = O.topk_experts(logits, k)
    for t in range(logits.shape[0]):
        assert list(idx[t]) == brute_topk(list(logits[t]), k), t


def test_topk_continuous_values():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((200, 8)).astype(np.float32).astype(np.float64)
    idx = O.topk_experts(logits, 4)
    for t in range(200):
        assert list(idx[t]) == brute_topk(list(logits[t]), 4)


def test_all_equal_logits_pick_lowest_indices():
    idx, g = O.route(np.full((3, 8), 0.7), 4)
    assert (idx == np.arange(4)).all()
    np.testing.assert_array_equal(g, np.full((3, 4), 0.25))


def test_k_equals_E_is_plain_softmax_sorted():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((10, 6))
    idx, g = O.route(l, 6)
    p = sp_softmax(l, axis=1)
    for t in range(10):
        assert sorted(idx[t]) == list(range(6))
        np.testing.assert_allclose(g[t], p[t, idx[t]], rtol=1e-14)
        assert all(l[t, idx[t][j]] >= l[t, idx[t][j + 1]] for j in range(5))


def test_k1_gate_is_one():
    rng = np.random.default_rng(3)
    _, g = O.route(rng.standard_normal((50, 8)), 1)
    np.testing.assert_array_equal(g, np.ones((50, 1)))


def test_gates_equal_softmax_over_selected_logits():
    # Closed form: the full-softmax denominator cancels in the renormalisation.
    rng = np.random.default_rng(4)
    l = rng.standard_normal((100, 16)) * 3
    idx, g = O.route(l, 4)
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(g, sp_softmax(sel, axis=1), rtol=1e-13)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-14)
    # Decreasing logits give non-increasing gates.
    assert (np.diff(g, axis=1) <= 1e-15).all()


def test_gates_shift_invariant_and_large_logits():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((20, 8))
    _, g1 = O.route(l, 3)
    _, g2 = O.route(l + 700.0, 3)  # would overflow exp without max subtraction
    np.testing.assert_allclose(g1, g2, rtol=1e-12)


def test_two_expert_closed_form():
    # E=2, k=2: g0 = 1/(1+exp(l1-l0)) for the larger logit.
    l = np.array([[1.5, -0.5]])
    _, g = O.route(l, 2)
    assert abs(g[0, 0] - 1 / (1 + np.exp(-2.0))) < 1e-15


def test_router_logits_brute_force():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 7)); w = rng.standard_normal((7, 3))
    l = O.router_logits(x, w)
    for t, e in itertools.product(range(5), range(3)):
        assert abs(l[t, e] - sum(x[t, i] * w[i, e] for i in range(7))) < 1e-12
