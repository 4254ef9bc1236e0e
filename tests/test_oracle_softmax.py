"""Pins of the oracle's softmax decode (the comparison side of the EntmaxKV page,
§3 "Analyse Théorique" and §4 "Résultats") against what the mathematics fixes."""
import math

import numpy as np
from scipy.special import logsumexp, softmax as scipy_softmax

from oracle import entmax, softmax


def test_single_token_gives_its_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    lse, p, o = softmax.softmax_decode_heads(q, k, v, 0.5)
    np.testing.assert_array_equal(p, np.ones((3, 1)))
    np.testing.assert_allclose(o, np.repeat(v, 3, axis=0), rtol=0, atol=0)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]), rtol=1e-15)


def test_equal_scores_give_the_mean_and_log_n():
    rng = np.random.default_rng(2)
    n, d = 37, 16
    k = np.tile(rng.standard_normal((1, d)), (n, 1))
    v = rng.standard_normal((n, d))
    q = rng.standard_normal((2, d))
    lse, p, o = softmax.softmax_decode_heads(q, k, v, 1.0)
    np.testing.assert_allclose(p, np.full((2, n), 1.0 / n), rtol=1e-14)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (2, 1)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, q @ k[0] + math.log(n), rtol=1e-14)


def test_two_tokens_by_hand():
    # scores 0 and log 3: weights 1/4 and 3/4, lse = log 4
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[4.0], [8.0]])
    lse, p, o = softmax.softmax_decode_heads(np.array([[1.0]]), k, v, 1.0)
    np.testing.assert_allclose(p[0], [0.25, 0.75], rtol=1e-15)
    np.testing.assert_allclose(o[0], [7.0], rtol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(4.0), rtol=1e-15)


def test_library_softmax_and_logsumexp():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 32)) * 3
    k = rng.standard_normal((500, 32))
    v = rng.standard_normal((500, 32))
    lse, p, o = softmax.softmax_decode_heads(q, k, v, 0.25)
    for h in range(4):
        s = 0.25 * (k @ q[h])
        np.testing.assert_allclose(p[h], scipy_softmax(s), rtol=1e-12, atol=1e-300)
        assert abs(lse[h] - logsumexp(s)) <= 1e-12 * abs(logsumexp(s)) + 1e-14
        np.testing.assert_allclose(o[h], scipy_softmax(s) @ v, rtol=1e-11, atol=1e-13)
        assert abs(p[h].sum() - 1.0) < 1e-13


def test_shift_invariance():
    rng = np.random.default_rng(4)
    d = 8
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((50, d))
    v = rng.standard_normal((50, d))
    lse0, _, o0 = softmax.softmax_decode_heads(q, k, v, 1.0)
    # adding c * q/|q|^2 to every key shifts every score by exactly c
    c = 5.0
    k2 = k + c * q[0] / (q[0] @ q[0])
    lse1, _, o1 = softmax.softmax_decode_heads(q, k2, v, 1.0)
    np.testing.assert_allclose(lse1 - lse0, c, rtol=1e-12)
    np.testing.assert_allclose(o1, o0, rtol=1e-11, atol=1e-13)


def test_entmax_tends_to_softmax():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((300, 16))
    v = rng.standard_normal((300, 16))
    _, p_soft, _ = softmax.softmax_decode_heads(q, k, v, 1.0)
    s = k @ q[0]
    for a1 in (1e-2, 1e-3):
        _, p_ent = entmax.entmax_scores(s, 1.0 + a1)
        assert np.abs(p_ent - p_soft[0]).sum() <= 10 * a1


def test_dropped_mass_identity_and_error_bound():
    """delta = 1 - exp(lse_I - lse_all) equals the full weights outside I; the kept
    weights renormalised differ from the full ones by exactly 2 delta in L1, so the
    output moves by at most 2 B delta (§3)."""
    rng = np.random.default_rng(6)
    n, d = 400, 24
    q = rng.standard_normal((3, d)) * 1.5
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    lse_all, p_all, o_all = softmax.softmax_decode_heads(q, k, v, 0.5)
    B = np.sqrt((v * v).sum(axis=1)).max()
    for trial in range(5):
        keep = rng.random(n) < 0.3 + 0.1 * trial
        lse_i, p_i, o_i = softmax.softmax_decode_heads(q, k[keep], v[keep], 0.5)
        delta = softmax.dropped_mass(lse_i, lse_all)
        np.testing.assert_allclose(delta, p_all[:, ~keep].sum(axis=1), rtol=1e-11, atol=1e-15)
        assert np.all(delta > 0)
        for h in range(3):
            full_on_keep = np.zeros(n)
            full_on_keep[keep] = p_i[h]
            l1 = np.abs(full_on_keep - p_all[h]).sum()
            assert abs(l1 - 2 * delta[h]) <= 1e-12
            assert np.linalg.norm(o_i[h] - o_all[h]) <= 2 * B * delta[h] * (1 + 1e-12)
