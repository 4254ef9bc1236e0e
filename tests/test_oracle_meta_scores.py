"""Pins of the oracle's page metadata and page scores.

EntmaxKV summary page, §2.A "Notation de Page Consciente de la Requête":
per-page bounding box (k_min, k_max) giving a deterministic upper bound on the
best score of any token of the page, and per-page key mean/variance giving a
Gaussian model of the page's scores.
"""
import math

import numpy as np
import pytest

from oracle import meta, scores


def _bf16_round(x):
    """Round-to-nearest-even to bf16, returned as exact fp64 (test data helper)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("seed", range(8))
def test_bbox_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(1, 40)), int(rng.integers(1, 20))
    k = _bf16_round(rng.normal(0, 3, (n, d)))
    kmin, kmax, _, _ = meta.page_meta(k)
    for j in range(d):
        assert all(kmin[j] <= k[i, j] <= kmax[j] for i in range(n))
        assert any(k[i, j] == kmin[j] for i in range(n))
        assert any(k[i, j] == kmax[j] for i in range(n))


@pytest.mark.parametrize("n,m", [(16, 3), (16, 8), (7, 1), (32, 31), (2, 1)])
def test_moments_closed_form(n, m):
    # column j takes value a_j on m tokens and b_j on the rest:
    # mean = (m a + (n-m) b)/n, population variance = m (n-m) (a-b)^2 / n^2
    rng = np.random.default_rng(n * 100 + m)
    d = 9
    a = _bf16_round(rng.normal(0, 2, d))
    b = _bf16_round(rng.normal(0, 2, d))
    k = np.empty((n, d))
    rows = rng.permutation(n)
    k[rows[:m]] = a
    k[rows[m:]] = b
    _, _, mu, var = meta.page_meta(k)
    mu_ref = (m * a + (n - m) * b) / n
    var_ref = m * (n - m) * (a - b) ** 2 / n ** 2
    np.testing.assert_array_equal(mu, mu_ref.astype(np.float32))
    np.testing.assert_allclose(var.astype(np.float64), var_ref, rtol=2 ** -23, atol=0)


def test_single_token_page():
    k = _bf16_round(np.array([[1.5, -2.0, 0.0, 3.25]]))
    kmin, kmax, mu, var = meta.page_meta(k)
    np.testing.assert_array_equal(kmin, k[0])
    np.testing.assert_array_equal(kmax, k[0])
    np.testing.assert_array_equal(mu, k[0].astype(np.float32))
    np.testing.assert_array_equal(var, np.zeros(4, np.float32))


def test_fast_matches_plain():
    rng = np.random.default_rng(5)
    k = _bf16_round(rng.normal(0, 1, (6, 16, 32)))
    fast = meta.page_meta_fast(k)
    for p in range(6):
        plain = meta.page_meta(k[p])
        np.testing.assert_array_equal(fast[0][p], plain[0])
        np.testing.assert_array_equal(fast[1][p], plain[1])
        np.testing.assert_array_equal(fast[2][p], plain[2])
        np.testing.assert_allclose(fast[3][p], plain[3], rtol=2 ** -23)


def test_box_bound_hand_case():
    # q = (1, -2); kmin = (-1, -1), kmax = (3, 0.5):
    # coordinate 0: max(-1, 3) = 3; coordinate 1: max(2, -1) = 2 -> 5
    q = np.array([1.0, -2.0])
    assert scores.box_bound(q, [-1.0, -1.0], [3.0, 0.5], 1.0) == np.float32(5.0)
    assert scores.box_bound(q, [-1.0, -1.0], [3.0, 0.5], 0.5) == np.float32(2.5)
    # all-negative query picks kmin everywhere
    assert scores.box_bound(np.array([-1.0, -1.0]), [-1.0, 2.0], [4.0, 3.0], 1.0) == np.float32(-1.0)


@pytest.mark.parametrize("seed", range(10))
def test_box_bound_dominates_every_token(seed):
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(1, 33)), 64
    k = _bf16_round(rng.normal(0, 1, (n, d)))
    q = rng.normal(0, 0.2, d).astype(np.float32).astype(np.float64)
    kmin, kmax, _, _ = meta.page_meta(k)
    u = scores.box_bound(q, kmin, kmax, 1.0)
    for i in range(n):
        s = math.fsum(q * k[i])
        assert u >= np.float32(s)
    if n == 1:
        assert u == np.float32(math.fsum(q * k[0]))


def test_box_bound_is_tight_for_corner_token():
    # a page containing the corner that maximises the bound attains it exactly
    rng = np.random.default_rng(11)
    d = 32
    k = _bf16_round(rng.normal(0, 1, (10, d)))
    q = rng.normal(0, 1, d).astype(np.float32).astype(np.float64)
    corner = np.where(q >= 0, k.max(axis=0), k.min(axis=0))
    k2 = np.vstack([k, corner])
    kmin, kmax, _, _ = meta.page_meta(k2)
    assert scores.box_bound(q, kmin, kmax, 1.0) == np.float32(math.fsum(q * corner))


def test_gauss_moments_match_sampling():
    # keys with independent coordinates N(mu_j, s2_j): the score <q,k> has mean
    # sum q mu and variance sum q^2 s2; check against a large sample
    rng = np.random.default_rng(12)
    d = 24
    mu = rng.normal(0, 1, d).astype(np.float32)
    s2 = rng.uniform(0.1, 2, d).astype(np.float32)
    q = rng.normal(0, 0.5, d).astype(np.float32).astype(np.float64)
    m, v = scores.gauss_moments(q, mu, s2, 1.0)
    ks = rng.normal(mu.astype(np.float64), np.sqrt(s2.astype(np.float64)), (400000, d))
    sc = ks @ q
    assert abs(sc.mean() - m) < 5 * math.sqrt(v / sc.size)
    assert abs(sc.var() - v) < 0.02 * v
    m2, v2 = scores.gauss_moments(q, mu, s2, 0.5)
    assert abs(m2 - 0.5 * m) < 1e-12 * (1 + abs(m)) and abs(v2 - 0.25 * v) < 1e-12 * v
