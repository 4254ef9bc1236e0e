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


def _bf16_values(x32):
    # a float32 holds a bf16 value iff its low 16 bits are zero
    return (np.asarray(x32, np.float32).view(np.uint32) & 0xFFFF) == 0


def test_round_bf16_hand_cases():
    r = meta.round_bf16
    e = 2.0 ** -7                        # bf16 spacing in [1, 2)
    assert r(1.0) == 1.0 and r(0.0) == 0.0 and r(-2.5) == -2.5
    assert r(1 + e / 2) == 1.0           # tie between 1 and 1 + e -> even (1)
    assert r(1 + 3 * e / 2) == 1 + 2 * e  # tie between 1 + e (odd) and 1 + 2e (even)
    assert r(1 + e / 2 + 2.0 ** -40) == 1 + e   # just above the tie
    # rounding through fp32 first would land on the tie and then go to 1.0
    x = 1 + e / 2 + 2.0 ** -30
    assert float(np.float32(x)) == 1 + e / 2
    assert r(x) == 1 + e
    assert r(-(1 + e / 2 + 2.0 ** -30)) == -(1 + e)
    # the spacing below 2^-126 stays 2^-133
    assert r(2.0 ** -133 * 5.5) == 2.0 ** -133 * 6
    assert r(2.0 ** -133 * 0.5) == 0.0
    assert r(255.5 * 2.0 ** -7) == 2.0          # carries into the next binade


def test_round_bf16_is_nearest_on_random_values():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 1, 20000) * np.exp2(rng.integers(-40, 40, 20000))
    r = meta.round_bf16(x)
    assert np.all(_bf16_values(r.astype(np.float32)))
    assert np.array_equal(r.astype(np.float32).astype(np.float64), r)
    # no bf16 value lies closer: compare with both neighbours of r
    _, ex = np.frexp(np.abs(r))
    sp = np.ldexp(1.0, np.maximum(ex - 8, -133))    # spacing above |r| ...
    sp_lo = np.where(np.abs(r) == np.ldexp(0.5, ex), sp / 2, sp)   # ... and below at a power of 2
    d = np.abs(x - r)
    up = np.abs(x - (r + np.sign(x) * sp))
    dn = np.abs(x - (r - np.sign(x) * sp_lo))
    assert np.all(d <= up) and np.all(d <= dn)


def test_bf16_moments_are_rounded_fp64_moments():
    rng = np.random.default_rng(8)
    keys = rng.normal(0, 1, (16, 64)).astype(np.float32).astype(np.float64)
    kmin, kmax, mu32, var32 = meta.page_meta(keys, "f32")
    kmin2, kmax2, mu16, var16 = meta.page_meta(keys, "bf16")
    assert np.array_equal(kmin, kmin2) and np.array_equal(kmax, kmax2)
    assert np.all(_bf16_values(mu16)) and np.all(_bf16_values(var16))
    mu64 = keys.mean(axis=0)
    var64 = ((keys - mu64) ** 2).mean(axis=0)
    # within half a bf16 spacing of the fp64 moments
    for a, b in ((mu16, mu64), (var16, var64)):
        _, ex = np.frexp(np.abs(b))
        assert np.all(np.abs(a - b) <= np.ldexp(1.0, ex - 9) * (1 + 1e-12))
    kminf, kmaxf, muf, varf = meta.page_meta_fast(keys[None], "bf16")
    assert np.array_equal(muf[0], mu16) and np.array_equal(varf[0], var16)
