"""Pins of the oracle's page selection policies.

EntmaxKV summary page, §2.B "Politiques de Sélection des Candidats": top-k on
the box bounds, and the Gaussian-aware estimate tau-hat of the entmax
threshold with margin Delta.
"""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle import select

from test_oracle_entmax import entmax15_sort, sparsemax_sort


def _rank_rule(U, k):
    # page p is selected iff fewer than k pages precede it in the order
    # (larger U first, then smaller index)
    n = len(U)
    out = []
    for p in range(n):
        before = sum(1 for r in range(n) if U[r] > U[p] or (U[r] == U[p] and r < p))
        if before < k:
            out.append(p)
    return out


@pytest.mark.parametrize("seed", range(10))
def test_topk_rank_rule(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    # coarse values force many exact ties
    U = np.round(rng.normal(0, 3, n) * 2) / 2
    U = U.astype(np.float32)
    for k in (1, 2, 5, n // 2 + 1, n, n + 7):
        assert select.topk_pages(U, k) == _rank_rule(U, k)


def test_topk_ties_and_overflow():
    U = np.ones(10, np.float32)
    assert select.topk_pages(U, 3) == [0, 1, 2]
    assert select.topk_pages(U, 50) == list(range(10))
    U = np.array([1, 5, 5, 2, 5, -1], np.float32)
    assert select.topk_pages(U, 2) == [1, 2]
    assert select.topk_pages(U, 4) == [1, 2, 3, 4]
    with pytest.raises(ValueError):
        select.topk_pages(U, 0)


@pytest.mark.parametrize("g", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("h", [-6.0, -3.0, -1.0, 0.0, 0.7, 2.0, 5.0])
def test_partial_moments_vs_quadrature(g, h):
    f = lambda z: (z + h) ** g * math.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    ref, _ = integrate.quad(f, -h, np.inf, epsabs=1e-300, epsrel=1e-13, limit=200)
    got = float(select.partial_moment(h, g))
    # the recurrence cancels in the left tail: relative accuracy drops there but
    # the absolute error (what matters inside a sum that equals 1) stays ~1e-16
    assert abs(got - ref) <= 1e-12 * abs(ref) + 1e-16, (got, ref)
    if h >= -1.0:
        assert abs(got - ref) <= 1e-13 * abs(ref) + 1e-300, (got, ref)


def _expand(mu_z, counts):
    return np.repeat(np.asarray(mu_z, float), counts)


@pytest.mark.parametrize("seed", range(6))
def test_tau_hat_zero_variance_is_exact_threshold(seed):
    # with zero variance every token of page p has z = mu_z[p]; F is then the
    # exact entmax normalisation of the expanded multiset
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    mu_z = rng.normal(0, 1.5, n)
    counts = rng.integers(1, 17, n)
    sig = np.zeros(n)
    t1 = select.gauss_tau_hat(mu_z, sig, counts, 1)
    assert abs(t1 - sparsemax_sort(_expand(mu_z, counts))) < 1e-12 * max(1, abs(t1))
    t2 = select.gauss_tau_hat(mu_z, sig, counts, 2)
    assert abs(t2 - entmax15_sort(_expand(mu_z, counts))) < 1e-12 * max(1, abs(t2))


@pytest.mark.parametrize("g", [1, 2, 4])
@pytest.mark.parametrize("seed", range(4))
def test_tau_hat_solves_normalisation(g, seed):
    rng = np.random.default_rng(50 + seed)
    n = 500
    mu_z = rng.normal(0, 1, n)
    sig = rng.uniform(0.0, 1.0, n)
    sig[::7] = 0.0
    counts = np.full(n, 16)
    t = select.gauss_tau_hat(mu_z, sig, counts, g)
    assert abs(select.gauss_F(t, mu_z, sig, counts, g) - 1.0) < 1e-12
    # F is decreasing: a little to the left is above 1, to the right below
    assert select.gauss_F(t - 1e-6, mu_z, sig, counts, g) > 1.0
    assert select.gauss_F(t + 1e-6, mu_z, sig, counts, g) < 1.0


def test_gauss_F_matches_monte_carlo():
    # F(tau) = sum_p n_p E[(X_p - tau)_+^g]: check one page by sampling
    rng = np.random.default_rng(9)
    mu, s, tau = 0.4, 0.7, 0.9
    x = rng.normal(mu, s, 2_000_000)
    for g in (1, 2, 4):
        mc = np.mean(np.maximum(x - tau, 0.0) ** g) * 16
        val = select.gauss_F(tau, [mu], [s], [16], g)
        assert abs(mc - val) < 0.01 * val


def test_gauss_select_threshold_rule_and_guard():
    # two heads; page kept iff (alpha-1) u >= tau_hat - delta for some head
    alpha, delta = 2.0, 0.1
    u = np.array([[0.0, 3.0, -1.0, 2.0], [0.5, -2.0, 2.5, 0.0]], np.float32)
    m = np.array([[0.0, 1.0, -1.0, 0.5], [0.2, -1.0, 1.0, 0.0]])
    v = np.zeros_like(m)
    counts = [16, 16, 16, 16]
    sel, taus = select.gauss_select(u, m, v, counts, alpha, delta)
    expect = [p for p in range(4) if any(u[h, p] >= taus[h] - delta for h in range(2))]
    assert sel == expect and len(sel) > 0
    # guard: bounds far below the estimate -> keep argmax U (lowest index on ties)
    u2 = np.array([[-5.0, -4.0, -4.0]], np.float32)
    m2 = np.array([[10.0, 10.0, 10.0]])
    sel2, _ = select.gauss_select(u2, m2, np.zeros_like(m2), [4, 4, 4], alpha, delta)
    assert sel2 == [1]


# Hand-worked box-bound rule away from alpha = 2, where (alpha-1) != 1.  All
# pages have zero variance and one valid token, so tau-hat is the exact entmax
# threshold of the page means in z-space: z = (alpha-1) m = [5, 0, 0.5, -1.5 or
# -1, 1]; only z = 5 lies above 4, and (5 - 4)^gamma = 1, so tau-hat = 4 for
# every gamma.  With Delta = 0.1 a page is kept iff (alpha-1) u >= 3.9.  Pages 1
# and 3 have u >= 3.9 but (alpha-1) u < 3.9 (dropped: an oracle that compared u
# itself would keep them); page 4 clears the bar by 0.005 in z-space (an oracle
# that scaled Delta by (alpha-1) would drop it).
@pytest.mark.parametrize("alpha,u,m", [
    (1.5, [10.5, 5.0, 8.0, 7.7, 7.81], [10.0, 0.0, 1.0, -3.0, 2.0]),
    (1.25, [20.5, 10.0, 16.0, 15.5, 15.7], [20.0, 0.0, 2.0, -4.0, 4.0]),
])
def test_gauss_select_hand_worked_alpha_scaling(alpha, u, m):
    u = np.array([u], np.float32)
    m = np.array([m])
    v = np.zeros_like(m)
    sel, taus = select.gauss_select(u, m, v, [1] * 5, alpha, 0.1)
    assert abs(taus[0] - 4.0) <= 1e-12
    assert sel == [0, 2, 4]
    # two heads: the union of the heads' kept pages.  The second head's means
    # are those of the first head shifted so that its own tau-hat is 4 - 2 = 2
    # and its bar 1.9; its bounds keep only page 1 ((alpha-1) * 4.0 / (alpha-1) = 4 >= 1.9)
    a1 = alpha - 1.0
    m2 = m[0] - 2.0 / a1
    u2 = np.full(5, 1.0, np.float32)
    u2[1] = np.float32(4.0 / a1)
    sel2, taus2 = select.gauss_select(np.stack([u[0], u2]), np.stack([m[0], m2]),
                                      np.zeros((2, 5)), [1] * 5, alpha, 0.1)
    assert abs(taus2[0] - 4.0) <= 1e-12 and abs(taus2[1] - 2.0) <= 1e-12
    assert sel2 == [0, 1, 2, 4]


# Expected maximum of n independent standard normals: closed forms for n <= 5
# (order statistics of the normal distribution): e_1 = 0, e_2 = 1/sqrt(pi),
# e_3 = 3/(2 sqrt(pi)), e_4 = 6/pi^(3/2) * arctan(sqrt(2)),
# e_5 = 5/(4 sqrt(pi)) * (1 + (6/pi) * arcsin(1/3)).
E_CLOSED = {
    1: 0.0,
    2: 1.0 / math.sqrt(math.pi),
    3: 3.0 / (2.0 * math.sqrt(math.pi)),
    4: 6.0 / math.pi ** 1.5 * math.atan(math.sqrt(2.0)),
    5: 5.0 / (4.0 * math.sqrt(math.pi)) * (1.0 + 6.0 / math.pi * math.asin(1.0 / 3.0)),
}


def test_expected_max_closed_forms():
    for n, e in E_CLOSED.items():
        assert abs(select.expected_max_std_normal(n) - e) <= 1e-13, n


def test_expected_max_monte_carlo_and_shape():
    rng = np.random.default_rng(17)
    for n in (16, 32):
        x = rng.standard_normal((200_000, n)).max(axis=1)
        mc, se = x.mean(), x.std() / math.sqrt(x.size)
        assert abs(select.expected_max_std_normal(n) - mc) < 5 * se, n
    es = [select.expected_max_std_normal(n) for n in range(1, 65)]
    assert all(b > a for a, b in zip(es, es[1:]))                      # increasing in n
    assert all(e < math.sqrt(2 * math.log(n)) for n, e in enumerate(es[1:], start=2))


def test_gauss_est_select_rule_and_guard():
    # est = m + e_n sqrt(v); keep iff (alpha-1) est >= tau_hat - delta for some head
    alpha, delta = 1.5, 0.05
    a1 = alpha - 1.0
    u = np.array([[4.0, 3.0, 2.0, 1.0], [1.0, 2.0, 3.0, 4.0]], np.float32)
    m = np.array([[6.0, 0.2, -0.5, 4.23], [0.1, 5.5, 3.0, -1.0]])
    v = np.array([[0.5, 2.0, 0.1, 1.0], [1.0, 0.3, 4.0, 0.2]])
    counts = [4, 4, 4, 3]                  # a ragged last page uses e_3
    sel, taus = select.gauss_est_select(u, m, v, counts, alpha, delta)
    e = np.array([E_CLOSED[c] for c in counts])
    expect = [p for p in range(4)
              if any(a1 * (m[h, p] + e[p] * math.sqrt(v[h, p])) >= taus[h] - delta
                     for h in range(2))]
    assert sel == expect == [0, 1, 2]
    # page 2 clears the bar only through its spread; page 3 would with e_4
    assert a1 * m[1, 2] < taus[1] - delta
    assert a1 * (m[0, 3] + E_CLOSED[4]) >= taus[0] - delta
    # the threshold is the Gaussian policy's own tau-hat
    _, taus_b = select.gauss_select(u, m, v, counts, alpha, delta)
    assert np.array_equal(taus, taus_b)
    # zero variance: the estimate is the mean itself
    sel0, t0 = select.gauss_est_select(u, m, np.zeros_like(v), counts, alpha, delta)
    assert sel0 == [p for p in range(4) if any(a1 * m[h, p] >= t0[h] - delta for h in range(2))]
    # guard: single-token pages (e_1 = 0) with a wide spread push tau-hat above
    # every estimate, so nothing clears the bar -> argmax U, lowest index on ties
    u2 = np.array([[1.0, 7.0, 7.0]], np.float32)
    m2 = np.zeros((1, 3))
    v2 = np.full((1, 3), 4.0)
    sel2, t2 = select.gauss_est_select(u2, m2, v2, [1, 1, 1], 2.0, 0.1)
    assert t2[0] - 0.1 > 0.0 and sel2 == [1]


@pytest.mark.parametrize("seed", range(4))
def test_page_masses_zero_variance_are_exact_entmax_masses(seed):
    # zero variance: each page's tokens all score mu_z[p]; the exact entmax
    # weights of the expanded multiset come from the sort-based closed forms,
    # and a page's mass is the sum of its tokens' weights
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(2, 40))
    mu_z = rng.normal(0, 1.5, n)
    counts = rng.integers(1, 17, n)
    sig = np.zeros(n)
    for g, closed in ((1, sparsemax_sort), (2, entmax15_sort)):
        tau_exact = closed(_expand(mu_z, counts))
        w = np.maximum(_expand(mu_z, counts) - tau_exact, 0.0) ** g
        per_page = np.add.reduceat(w, np.concatenate([[0], np.cumsum(counts)[:-1]]))
        t = select.gauss_tau_hat(mu_z, sig, counts, g)
        M = select.gauss_page_masses(mu_z, sig, counts, g, t)
        np.testing.assert_allclose(M, per_page, rtol=1e-9, atol=1e-12)
        assert abs(math.fsum(M) - 1.0) < 1e-12


def test_page_masses_monte_carlo_and_sum():
    rng = np.random.default_rng(11)
    mu, s, tau, cnt = -0.3, 0.9, 0.2, 16
    x = rng.normal(mu, s, 2_000_000)
    for g in (1, 2, 3):
        mc = cnt * np.mean(np.maximum(x - tau, 0.0) ** g)
        val = select.gauss_page_masses([mu], [s], [cnt], g, tau)[0]
        assert abs(mc - val) < 0.01 * val
    # at tau-hat the masses of all pages sum to 1
    n = 300
    mu_z = rng.normal(0, 1, n)
    sig = rng.uniform(0.0, 1.2, n)
    sig[::5] = 0.0
    counts = rng.integers(1, 17, n)
    for g in (1, 2, 4):
        t = select.gauss_tau_hat(mu_z, sig, counts, g)
        assert abs(math.fsum(select.gauss_page_masses(mu_z, sig, counts, g, t)) - 1.0) < 1e-12


def test_gauss_mass_select_rule_and_guard():
    # keep p iff n_p E[(X - tau_hat)_+^g] >= eps for some head; a page whose mean
    # lies below tau-hat can still carry mass through its spread
    alpha, eps = 1.5, 0.02
    a1, g = alpha - 1.0, 2
    u = np.array([[4.0, 3.0, 2.0, 1.0], [1.0, 2.0, 3.0, 4.0]], np.float32)
    m = np.array([[6.0, 0.2, -0.5, 4.23], [0.1, 5.5, 3.0, -1.0]])
    v = np.array([[0.5, 2.0, 0.1, 1.0], [1.0, 0.3, 9.0, 0.2]])
    counts = [4, 4, 4, 3]
    sel, taus = select.gauss_mass_select(u, m, v, counts, alpha, eps)
    M = np.array([select.gauss_page_masses(a1 * m[h], a1 * np.sqrt(v[h]), counts, g, taus[h])
                  for h in range(2)])
    expect = [p for p in range(4) if (M[:, p] >= eps).any()]
    assert sel == expect and len(sel) >= 2
    assert a1 * m[1, 2] < taus[1] and M[1, 2] >= eps        # kept through its spread
    # the threshold is the Gaussian policy's own tau-hat
    _, taus_b = select.gauss_select(u, m, v, counts, alpha, eps)
    assert np.array_equal(taus, taus_b)
    # a larger threshold keeps a subset
    sel_hi, _ = select.gauss_mass_select(u, m, v, counts, alpha, 0.3)
    assert set(sel_hi) <= set(sel)
    # guard: no page holds more than mass 1, so eps > 1 keeps only argmax U
    # (lowest index on ties)
    u2 = np.array([[1.0, 7.0, 7.0]], np.float32)
    sel2, _ = select.gauss_mass_select(u2, np.zeros((1, 3)), np.ones((1, 3)), [4, 4, 4], 2.0, 1.5)
    assert sel2 == [1]


# ---- non-integer gamma (1 < alpha < 2): the quadrature of I_g ----

def _pcf_closed_form(h, g):
    # I_g(h) = Gamma(g+1) exp(-h^2/4) D_{-g-1}(-h) / sqrt(2 pi), parabolic
    # cylinder function D at 40 significant digits
    import mpmath
    with mpmath.workdps(40):
        h = mpmath.mpf(h)
        g = mpmath.mpf(g)
        v = mpmath.gamma(g + 1) * mpmath.exp(-h * h / 4) * mpmath.pcfd(-g - 1, -h)
        return float(v / mpmath.sqrt(2 * mpmath.pi))


@pytest.mark.parametrize("g", [1.0 / 0.7, 1.0 / 0.7 - 1.0, 2.5, 1.5, 0.5, 3.3])
@pytest.mark.parametrize("h", [-9.0, -5.0, -2.0, -0.5, 0.0, 0.3, 1.0, 2.5, 5.0, 8.0, 12.0])
def test_partial_moment_quadrature_vs_parabolic_cylinder(g, h):
    got = select.partial_moment_quad(h, g)
    ref = _pcf_closed_form(h, g)
    assert abs(got - ref) <= 1e-13 * abs(ref), (got, ref)


@pytest.mark.parametrize("g", [1, 2, 3, 4])
@pytest.mark.parametrize("h", [-6.0, -1.0, 0.0, 0.7, 2.0, 5.0])
def test_partial_moment_quadrature_matches_integer_recurrence(g, h):
    got = select.partial_moment_quad(h, float(g))
    ref = float(select.partial_moment(h, g))
    # (the recurrence loses relative accuracy in the left tail, as above)
    assert abs(got - ref) <= 1e-12 * abs(ref) + 1e-16, (g, h, got, ref)
    if h >= -1.0:
        assert abs(got - ref) <= 1e-13 * abs(ref), (g, h, got, ref)


@pytest.mark.parametrize("g", [1.0 / 0.7, 2.5, 1.0 / 0.55])
@pytest.mark.parametrize("h", [-3.0, -0.5, 0.0, 1.5, 4.0])
def test_partial_moment_quadrature_stein_recurrence(g, h):
    # E[(Z+h)_+^(g+1)] = h E[(Z+h)_+^g] + g E[(Z+h)_+^(g-1)] (Stein's identity)
    lhs = select.partial_moment_quad(h, g + 1.0)
    rhs = h * select.partial_moment_quad(h, g) + g * select.partial_moment_quad(h, g - 1.0)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs), (lhs, rhs)


def test_selection_gamma_rule():
    assert select.selection_gamma(1.5) == 2 and isinstance(select.selection_gamma(1.5), int)
    assert select.selection_gamma(2.0) == 1
    g = select.selection_gamma(1.7)
    assert isinstance(g, float) and abs(g - 1.0 / 0.7) < 1e-15
    assert abs(select.selection_gamma(1.4) - 2.5) < 1e-15
    for bad in (2.5, 1.0, 0.9, 3.0):
        with pytest.raises(ValueError):
            select.selection_gamma(bad)


@pytest.mark.parametrize("alpha", [1.7, 1.4])
@pytest.mark.parametrize("seed", range(3))
def test_tau_hat_fractional_zero_variance_is_exact_threshold(alpha, seed):
    # zero-variance pages: F is the exact entmax normalisation of the expanded
    # multiset, whose threshold the decode oracle finds on the tokens directly
    from oracle import entmax
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(2, 30))
    mu_z = rng.normal(0, 1.5, n)
    counts = rng.integers(1, 17, n)
    g = select.selection_gamma(alpha)
    t = select.gauss_tau_hat(mu_z, np.zeros(n), counts, g)
    ref = entmax.threshold(_expand(mu_z, counts), alpha)  # z-space scores
    assert abs(t - ref) < 1e-12 * max(1.0, abs(ref)), (t, ref)


@pytest.mark.parametrize("seed", range(2))
def test_tau_hat_fractional_solves_normalisation_and_is_continuous(seed):
    rng = np.random.default_rng(90 + seed)
    n = 24
    mu_z = rng.normal(0, 1, n)
    sig = rng.uniform(0.05, 1.0, n)
    sig[::5] = 0.0
    counts = rng.integers(1, 17, n)
    for g in (1.0 / 0.7, 2.5):
        t = select.gauss_tau_hat(mu_z, sig, counts, g)
        assert abs(select.gauss_F(t, mu_z, sig, counts, g) - 1.0) < 1e-12
        assert select.gauss_F(t - 1e-6, mu_z, sig, counts, g) > 1.0
        assert select.gauss_F(t + 1e-6, mu_z, sig, counts, g) < 1.0
    # gamma -> 1, 2 from either side: the quadrature path approaches the
    # integer recurrence's root (tau-hat is smooth in gamma)
    for gi in (1, 2):
        t0 = select.gauss_tau_hat(mu_z, sig, counts, gi)
        for eps in (1e-7, -1e-7):
            if gi == 1 and eps < 0:
                continue  # gamma < 1 is outside the reading
            t1 = select.gauss_tau_hat(mu_z, sig, counts, gi + eps)
            assert abs(t1 - t0) < 1e-5 * max(1.0, abs(t0)), (gi, eps, t0, t1)
