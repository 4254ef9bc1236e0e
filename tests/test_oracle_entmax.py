"""Pins of the oracle's alpha-entmax against what the mathematics fixes.

EntmaxKV summary page, §2 "Méthodologie": alpha-entmax (alpha > 1) gives exact
zeros; the threshold tau is global.  The closed forms below are independent
derivations (sorting + prefix sums), not the oracle's bisection.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

from oracle import entmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "entmax_hand.json")


def sparsemax_sort(z):
    """Sort-based sparsemax (alpha = 2): k* = max{k : 1 + k z_(k) > sum_{j<=k} z_(j)}."""
    zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
    cs = np.cumsum(zs)
    k = np.arange(1, zs.size + 1)
    ok = 1.0 + k * zs > cs
    kstar = int(k[ok].max())
    return (cs[kstar - 1] - 1.0) / kstar


def entmax15_sort(z):
    """1.5-entmax (gamma = 2) by sorting: per prefix k, tau_k = mu_k - sqrt((1 - k var_k)/k),
    and tau = tau_{k*} for the largest k with tau_k <= z_(k)."""
    zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
    best = None
    for k in range(1, zs.size + 1):
        top = zs[:k]
        mu = top.mean()
        var = ((top - mu) ** 2).mean()
        disc = (1.0 - k * var) / k
        if disc < 0:
            break
        tk = mu - math.sqrt(disc)
        if tk <= zs[k - 1]:
            best = tk
    return best


def test_hand_worked_cases():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 6
    for c in cases:
        z = np.array(c["z"])
        tau = entmax.threshold(z, c["alpha"])
        p = entmax.weights(z, tau, c["alpha"])
        assert abs(tau - c["tau"]) <= 1e-12, c
        np.testing.assert_allclose(p, c["p"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("n", [1, 2, 7, 64, 1000])
def test_alpha2_matches_sort_closed_form(seed, n):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1 + seed, n)
    tau = entmax.threshold(z, 2.0)
    assert abs(tau - sparsemax_sort(z)) <= 1e-12 * max(1.0, abs(tau))
    p = entmax.weights(z, tau, 2.0)
    ref = np.maximum(z - sparsemax_sort(z), 0.0)
    np.testing.assert_allclose(p, ref, atol=1e-12)


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("n", [1, 3, 50, 600])
def test_alpha15_matches_quadratic_closed_form(seed, n):
    rng = np.random.default_rng(100 + seed)
    z = rng.normal(0, 0.3 * (1 + seed), n)
    tau = entmax.threshold(z, 1.5)
    assert abs(tau - entmax15_sort(z)) <= 1e-12 * max(1.0, abs(tau))


@pytest.mark.parametrize("alpha,tol", [(1.1, 1.0), (1.01, 0.1), (1.001, 0.01)])
def test_alpha_to_one_tends_to_softmax(alpha, tol):
    rng = np.random.default_rng(7)
    s = rng.normal(0, 1, 1000)
    tau, p = entmax.entmax_scores(s, alpha)
    l1 = np.abs(p - scipy_softmax(s)).sum()
    assert l1 <= 10 * (alpha - 1), l1


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0, 2.5, 3.0])
@pytest.mark.parametrize("seed", range(6))
def test_invariants(alpha, seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 3000))
    z = rng.normal(0, float(rng.uniform(0.01, 20)), n)
    tau = entmax.threshold(z, alpha)
    p = entmax.weights(z, tau, alpha)
    assert abs(math.fsum(p) - 1.0) <= 1e-12
    # exact zeros off the support, strictly positive on it
    assert np.all(p[z <= tau] == 0.0)
    assert np.all(p[z > tau] > 0.0)
    # bracket derived from the definition
    zmax = z.max()
    assert zmax - 1.0 <= tau <= zmax - n ** (1.0 - alpha) + 1e-15
    assert p.max() <= 1.0 + 1e-15


def test_absent_tokens_are_ignored():
    z = np.array([0.3, -np.inf, 1.2, -np.inf, 0.9])
    tau = entmax.threshold(z, 2.0)
    assert abs(tau - sparsemax_sort(z[np.isfinite(z)])) < 1e-13
    p = entmax.weights(z, tau, 2.0)
    assert p[1] == 0.0 and p[3] == 0.0
    assert abs(p.sum() - 1.0) < 1e-13


def test_shift_invariance():
    # adding a constant to every z shifts tau by that constant and leaves p unchanged
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, 500)
    for alpha in (1.5, 2.0, 1.25):
        t0 = entmax.threshold(z, alpha)
        t1 = entmax.threshold(z + 37.0, alpha)
        assert abs((t1 - 37.0) - t0) < 1e-11
        np.testing.assert_allclose(entmax.weights(z, t0, alpha), entmax.weights(z + 37.0, t1, alpha),
                                   atol=1e-10)


def test_rejects_alpha_le_one():
    with pytest.raises(ValueError):
        entmax.threshold(np.zeros(3), 1.0)
