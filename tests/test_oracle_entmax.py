"""Pins of the oracle's alpha-entmax (Stage 1 of the DashAttention explainer,
w = alpha-entmax(gamma * zbar)) against what the mathematics fixes.

Reading: alpha-entmax is the Tsallis entmax, argmax_{p in simplex}
p.y + sum_j (p_j - p_j^alpha) / (alpha (alpha - 1)), whose solution is
p_j = [(alpha-1) y_j - tau]_+^(1/(alpha-1)).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import minimize

import oracle
from brute import softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tsallis_slsqp(y, alpha):
    """Independent solve of the defining optimisation problem with SLSQP."""
    y = np.asarray(y, np.float64)
    n = len(y)

    def neg(p):
        p = np.clip(p, 0.0, None)
        return -(p @ y + np.sum(p - p ** alpha) / (alpha * (alpha - 1.0)))

    def grad(p):
        p = np.clip(p, 1e-300, None)
        return -(y + (1.0 - alpha * p ** (alpha - 1.0)) / (alpha * (alpha - 1.0)))

    best = None
    for start in (np.full(n, 1.0 / n), softmax(y)):
        res = minimize(neg, start, jac=grad, method="SLSQP", bounds=[(0.0, 1.0)] * n,
                       constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1.0,
                                     "jac": lambda p: np.ones_like(p)}],
                       options={"ftol": 1e-15, "maxiter": 2000})
        if best is None or res.fun < best.fun:
            best = res
    return np.clip(best.x, 0.0, None)


def test_golden_closed_forms():
    """Cases whose answers follow by hand from the KKT conditions (file cites
    the derivation of each)."""
    with open(os.path.join(GOLDEN, "entmax_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 6
    for c in cases:
        p, tau = oracle.entmax_of_scores(c["y"], c["alpha"])
        np.testing.assert_allclose(p, c["p"], rtol=0, atol=1e-12, err_msg=c["why"])
        assert abs(tau - c["tau"]) < 1e-12, c["why"]


@pytest.mark.parametrize("t", [-1.9, -1.0, -0.3, 0.0, 0.4, 1.0, 1.7, 1.99, 2.0, 3.5])
def test_entmax15_binary_closed_form(t):
    """1.5-entmax([t, 0]): both entries in the support solve
    (t/2 - tau)^2 + tau^2 = 1, i.e. tau = (t - sqrt(8 - t^2)) / 4 for |t| < 2,
    and p_1 = ((t + sqrt(8 - t^2)) / 4)^2; for t >= 2 the support is {1}."""
    p, tau = oracle.entmax_of_scores([t, 0.0], 1.5)
    if abs(t) < 2:
        p1 = ((t + math.sqrt(8 - t * t)) / 4) ** 2
        assert abs(tau - (t - math.sqrt(8 - t * t)) / 4) < 1e-12
        np.testing.assert_allclose(p, [p1, 1 - p1], atol=1e-12)
    else:
        np.testing.assert_allclose(p, [1.0, 0.0] if t > 0 else [0.0, 1.0], atol=1e-12)


@pytest.mark.parametrize("t", [-2.0, -0.999, -0.5, 0.0, 0.25, 0.9, 1.0, 4.0])
def test_sparsemax_binary_closed_form(t):
    """sparsemax([t, 0]) = [(1+t)/2, (1-t)/2] clipped to the simplex."""
    p, _ = oracle.entmax_of_scores([t, 0.0], 2.0)
    p1 = min(max((1 + t) / 2, 0.0), 1.0)
    np.testing.assert_allclose(p, [p1, 1 - p1], atol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0])
def test_matches_independent_slsqp(alpha):
    rng = np.random.default_rng(11)
    for n in (2, 3, 5, 8):
        for scale in (0.3, 1.0, 3.0):
            y = rng.standard_normal(n) * scale
            p, _ = oracle.entmax_of_scores(y, alpha)
            ref = tsallis_slsqp(y, alpha)
            np.testing.assert_allclose(p, ref, atol=2e-5, err_msg=f"y={y}")


def test_alpha_to_one_is_softmax():
    """As alpha -> 1 the Tsallis entropy tends to Shannon's and entmax to
    softmax, with an error that shrinks linearly in alpha - 1."""
    z = np.array([3.0, 1.0, 0.2, -1.0])
    errs = []
    for a in (1.1, 1.01, 1.001):
        p, _ = oracle.entmax_of_scores(z, a)
        errs.append(np.abs(p - softmax(z)).max())
    assert errs[0] > errs[1] > errs[2]
    assert 5 < errs[0] / errs[1] < 20 and 5 < errs[1] / errs[2] < 20
    assert errs[2] < 1e-3


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_invariants(alpha):
    rng = np.random.default_rng(5)
    e = 1.0 / (alpha - 1.0)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        x = rng.standard_normal(n) * rng.choice([0.05, 0.5, 2.0, 10.0])
        p, tau = oracle.entmax(x, alpha)
        assert np.all(p >= 0)
        assert abs(p.sum() - 1) < 1e-12
        # support is exactly {x > tau} and p follows the threshold form there
        assert np.array_equal(p > 0, x > tau)
        np.testing.assert_allclose(p[x > tau], (x[x > tau] - tau) ** e, rtol=1e-9)
        # tau lies in [max - 1, max - n^(1 - alpha)]
        assert x.max() - 1 - 1e-12 <= tau <= x.max() - n ** (1 - alpha) + 1e-12
        # shift invariance, permutation equivariance, monotonicity
        p2, tau2 = oracle.entmax(x + 0.37, alpha)
        np.testing.assert_allclose(p2, p, atol=1e-12)
        assert abs(tau2 - tau - 0.37) < 1e-9
        perm = rng.permutation(n)
        p3, _ = oracle.entmax(x[perm], alpha)
        np.testing.assert_allclose(p3, p[perm], atol=1e-12)
        order = np.argsort(x)
        assert np.all(np.diff(p[order]) >= -1e-15)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_special_inputs(alpha):
    for n in (1, 2, 7, 64):
        p, _ = oracle.entmax(np.full(n, 0.3), alpha)
        np.testing.assert_allclose(p, np.full(n, 1.0 / n), atol=1e-12)
    p, tau = oracle.entmax(np.array([2.5]), alpha)
    assert p[0] == 1.0 and abs(tau - 1.5) < 1e-12
    # one dominant score -> support {argmax}
    p, _ = oracle.entmax(np.array([0.0, 5.0, 0.1, -2.0]), alpha)
    np.testing.assert_allclose(p, [0, 1, 0, 0], atol=1e-15)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_sort_and_bisection_agree(alpha):
    rng = np.random.default_rng(9)
    for _ in range(100):
        x = rng.standard_normal(int(rng.integers(1, 200))) * rng.choice([0.1, 1.0, 5.0])
        p1, t1 = oracle.entmax(x, alpha)
        p2, t2 = oracle.entmax(x, alpha, method="bisect")
        assert abs(t1 - t2) < 1e-12
        np.testing.assert_allclose(p1, p2, atol=1e-12)
