"""Pins of the router oracle (oracle/router_oracle.py) against closed forms,
brute force and invariants; none re-types the oracle's formulas."""
import itertools
import math

import numpy as np
import pytest

from oracle import router_oracle as ro


def test_rms_norm_hand_example():
    # x = [1, 2, 3, 4]: mean of squares 7.5, so x_hat = x / sqrt(7.5) (eps 0, gamma 1)
    got = ro.rms_norm_rows(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), 0.0)
    assert np.allclose(got, np.array([[1, 2, 3, 4]]) / math.sqrt(7.5), rtol=1e-15)
    # gamma scales columns; eps enters under the root
    got = ro.rms_norm_rows(np.array([[3.0, -4.0]]), np.array([2.0, 0.5]), 0.5)
    assert np.allclose(got, np.array([[6.0, -2.0]]) / math.sqrt(12.5 + 0.5), rtol=1e-15)


def test_rms_norm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 64))
    a = ro.rms_norm_rows(x, np.ones(64), 0.0)
    b = ro.rms_norm_rows(7.25 * x, np.ones(64), 0.0)
    assert np.allclose(a, b, rtol=1e-13)
    assert np.allclose(np.sqrt(np.mean(a * a, axis=1)), 1.0, rtol=1e-13)


def test_top_k_brute_force_and_ties():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.integers(-3, 4, size=9).astype(np.float64)  # many ties
        k = int(rng.integers(1, 9))
        got = list(ro.top_k(z, k))
        # brute force: the lexicographically best k-tuple under (value desc, index asc)
        best = min(itertools.permutations(range(9), k), key=lambda p: [(-z[e], e) for e in p])
        assert got == list(best)


def test_activation_closed_forms():
    z = np.array([2.0, 0.0, -1.0])
    assert np.allclose(ro.activate_selected(z, ro.SIGMOID), [1 / (1 + math.e ** -2), 0.5, 1 / (1 + math.e)])
    s = ro.activate_selected(z, ro.SOFTMAX)
    den = math.e ** 2 + 1 + math.e ** -1
    assert np.allclose(s, [math.e ** 2 / den, 1 / den, math.e ** -1 / den], rtol=1e-15)
    # softmax is shift-invariant, sigmoid is not
    assert np.allclose(ro.activate_selected(z + 100.0, ro.SOFTMAX), s, rtol=1e-12)


def test_full_function_hand_example():
    # H = 4, E = 3: W picks x_hat[0], x_hat[3] and x_hat[1] - x_hat[2]
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    w = np.array([[1, 0, 0], [0, 0, 1], [0, 0, -1], [0, 1, 0]], dtype=np.float64)
    r = math.sqrt(7.5)
    xh, idx, aff = ro.rmsnorm_router_topk(x, np.ones(4), w, None, 0.0, 2, ro.SOFTMAX)
    logits = np.array([1 / r, 4 / r, -1 / r])
    assert list(idx[0]) == [1, 0]
    e1, e0 = math.exp(4 / r), math.exp(1 / r)
    assert np.allclose(aff[0], [e0 / (e0 + e1), e1 / (e0 + e1), 0.0], rtol=1e-14)
    assert aff[0, 2] == 0.0
    # a bias large enough moves expert 2 to the top, and the sigmoid sees the biased logit
    _, idx, aff = ro.rmsnorm_router_topk(x, np.ones(4), w, np.array([0.0, 0.0, 2.0]), 0.0, 1, ro.SIGMOID)
    assert list(idx[0]) == [2]
    assert np.isclose(aff[0, 2], 1 / (1 + math.exp(-(logits[2] + 2.0))), rtol=1e-14)


def test_expert_permutation_equivariance():
    rng = np.random.default_rng(2)
    T, H, E, K = 4, 32, 16, 4
    x, g = rng.standard_normal((T, H)), 1 + 0.1 * rng.standard_normal(H)
    w, b = rng.standard_normal((H, E)), rng.standard_normal(E)
    perm = rng.permutation(E)
    _, i1, a1 = ro.rmsnorm_router_topk(x, g, w, b, 1e-6, K, ro.SIGMOID)
    _, i2, a2 = ro.rmsnorm_router_topk(x, g, w[:, perm], b[perm], 1e-6, K, ro.SIGMOID)
    assert np.array_equal(perm[i2], i1)
    assert np.allclose(a2, a1[:, perm], rtol=1e-13)


@pytest.mark.parametrize("act", [ro.SIGMOID, ro.SOFTMAX])
def test_masked_affinities_structure(act):
    rng = np.random.default_rng(3)
    x, w = rng.standard_normal((5, 64)), rng.standard_normal((64, 32))
    _, idx, aff = ro.rmsnorm_router_topk(x, np.ones(64), w, None, 1e-6, 6, act)
    for t in range(5):
        assert np.count_nonzero(aff[t]) == 6 and set(np.flatnonzero(aff[t])) == set(idx[t])
        if act == ro.SOFTMAX:
            assert math.isclose(aff[t].sum(), 1.0, rel_tol=1e-13)
        # descending logits give descending affinities (both activations are monotone)
        assert np.all(np.diff(aff[t, idx[t]]) <= 0)
