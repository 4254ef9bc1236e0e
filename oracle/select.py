"""Candidate page selection, in fp64 (oracle; test infrastructure).

EntmaxKV page, §2.B "Politiques de Sélection des Candidats", two policies:

1. Top-k pages: a fixed budget, the k pages with the highest bounding-box
   upper bounds.  Readings: per (row, KV head) the group's bound
   U_p = max over the group's query heads of u_{h,p}; ranked on the fp32 U;
   equal U go to the lowest logical page index; k >= n selects every page;
   the result is returned in ascending page order.

2. Gaussian-aware entmax selection: estimate the global entmax threshold from
   the per-page Gaussian statistics by solving an approximate normalisation for
   tau-hat, then keep the pages whose estimated maximum score clears tau-hat
   lowered by a safety margin Delta.  Readings:
     * approximate normalisation, per query head h (z-space):
         F_h(tau) = sum_p n_p * E[(X_p - tau)_+^gamma] = 1,
         X_p ~ N((alpha-1) m_{h,p}, (alpha-1)^2 v_{h,p}),
       i.e. each page's token sum is replaced by its valid-token count times the
       Gaussian expectation of one token's entmax weight;
     * the page's "estimated maximum score" is its box bound, so page p is kept
       when (alpha-1) u_{h,p} >= tau-hat_h - Delta for some head h of the group
       (Delta in z-space units);
     * if no page clears the bar, the page with the largest U is kept (ties to
       the lowest index), so the entmax input is never empty.
   A second reading of the "estimated maximum score" (policy G-est) takes the
   page's n_p token scores as n_p independent draws from N(m_{h,p}, v_{h,p})
   and estimates their maximum by its expectation,
         est_{h,p} = m_{h,p} + e_{n_p} sqrt(v_{h,p}),
         e_n = E[max of n iid N(0, 1)] = integral of x n phi(x) Phi(x)^(n-1) dx,
   and keeps p when (alpha-1) est_{h,p} >= tau-hat_h - Delta for some head h
   of the group, with the same tau-hat and the same empty-set guard.

A third reading (policy G-mass) tests each page's expected mass instead of
its maximum: under the same model the tokens of page p carry, for head h, the
expected entmax mass
      M_{h,p} = n_p * E[(X_{h,p} - tau-hat_h)_+^gamma],
and these masses sum to F_h(tau-hat_h) = 1 over the pages.  Dropping a page
drops its mass, and the output error is at most 2 B times the dropped mass
(§3), so page p is kept when M_{h,p} >= eps for some head h of the group
(eps is the policy's threshold; same tau-hat, same empty-set guard).

Gaussian partial moments, I_g(h) = E[(Z + h)_+^g] for Z ~ N(0, 1):
   I_0 = Phi(h),  I_1 = h Phi(h) + phi(h),  I_g = h I_{g-1} + (g-1) I_{g-2}
(the last by Stein's identity E[Z f(Z)] = E[f'(Z)]), and for X ~ N(mu, s^2),
   E[(X - c)_+^g] = s^g I_g((mu - c)/s).
For a gamma that is not an integer (1 < alpha < 2, alpha not 1 + 1/n) the
oracle evaluates the defining integral I_g(h) = int_0^inf x^g phi(x - h) dx by
adaptive quadrature.  The reading stops at alpha <= 2 (gamma >= 1): F_h is
then convex as well as decreasing, and the solvers (the oracle's bisection and
the device's monotone Newton) are defined on that range only.
F_h is continuous and decreasing; at tau = max_p (alpha-1) m_{h,p} - 1 the page
with the largest mean alone contributes at least 1 (Jensen, x -> x_+^g being
convex for g >= 1), so F_h >= 1 there.

Pins (tests/test_oracle_select.py): top-k against a brute-force full sort and
hand-built tie cases; e_n against the closed forms known for n <= 5 and a
Monte Carlo estimate; I_g against numerical quadrature (scipy.integrate.quad);
for non-integer g, the quadrature against the parabolic-cylinder closed form
I_g(h) = Gamma(g+1) e^(-h^2/4) D_{-g-1}(-h) / sqrt(2 pi) (mpmath, 40 digits),
against the integer recurrence when g is an integer, and against Stein's
recurrence between g - 1, g and g + 1; tau-hat for non-integer g approaches
the integer-g solutions as g -> 1, 2 and, for zero-variance pages, equals the
exact entmax threshold (oracle.entmax.threshold) of the expanded multiset;
tau-hat for zero-variance pages equals the exact entmax threshold of the
expanded token multiset (checked against the sort-based sparsemax closed form);
the box-bound keep rule on hand-worked pages at alpha = 1.5 and 1.25 (literal
page lists; pages with u >= tau-hat - Delta > (alpha-1) u must be dropped);
F(tau-hat) = 1; page masses: for zero-variance pages they are the exact entmax
masses of the pages' tokens, and one page's expected mass matches a Monte
Carlo estimate.
"""
from __future__ import annotations

import math

import warnings

import numpy as np
from scipy import integrate
from scipy.special import ndtr


def topk_pages(U, k: int):
    """Ascending page indices of the min(k, n) largest fp32 bounds (ties: lowest index)."""
    U = np.asarray(U, dtype=np.float32)
    n = U.size
    if k < 1:
        raise ValueError("top-k needs k >= 1")
    order = sorted(range(n), key=lambda p: (-float(U[p]), p))
    return sorted(order[: min(k, n)])


def partial_moment(h, g: int):
    """I_g(h) = E[(Z + h)_+^g], Z standard normal, integer g >= 0 (vectorised in h)."""
    h = np.asarray(h, dtype=np.float64)
    Phi = ndtr(h)
    phi = np.exp(-0.5 * h * h) / math.sqrt(2.0 * math.pi)
    if g == 0:
        return Phi
    i_prev, i_cur = Phi, h * Phi + phi
    for k in range(2, g + 1):
        i_prev, i_cur = i_cur, h * i_cur + (k - 1) * i_prev
    return i_cur


def selection_gamma(alpha: float):
    """gamma = 1/(alpha-1) for the Gaussian rules: an int when it is one (to
    within 1e-6 relative, the integer recurrence), else the float; alpha must
    lie in (1, 2] (gamma >= 1)."""
    a = float(alpha)
    if not (1.0 < a <= 2.0):
        raise ValueError("the Gaussian rules are read for 1 < alpha <= 2 (gamma >= 1)")
    g = 1.0 / (a - 1.0)
    gi = int(round(g))
    if abs(g - gi) <= 1e-6 * gi:
        return gi
    return g


def partial_moment_quad(h: float, g: float) -> float:
    """I_g(h) = int_0^inf x^g phi(x - h) dx by adaptive quadrature (any real g > -1)."""
    h = float(h)
    g = float(g)

    def f(x):
        return x ** g * math.exp(-0.5 * (x - h) * (x - h)) / math.sqrt(2.0 * math.pi)

    # the integrand is negligible beyond max(h, 0) + 40; split at its peak
    top = max(h, 0.0) + 40.0
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", integrate.IntegrationWarning)
        if h > 0.0:
            a = integrate.quad(f, 0.0, h, epsabs=0.0, epsrel=2e-14, limit=500)[0]
            b = integrate.quad(f, h, top, epsabs=0.0, epsrel=2e-14, limit=500)[0]
            return a + b
        return integrate.quad(f, 0.0, top, epsabs=0.0, epsrel=2e-14, limit=500)[0]


def partial_moment_real(h, g):
    """I_g(h) for a real g >= 0: the integer recurrence for an int g, else
    quadrature of the definition (vectorised in h)."""
    if isinstance(g, (int, np.integer)):
        return partial_moment(h, int(g))
    h = np.asarray(h, dtype=np.float64)
    out = np.array([partial_moment_quad(x, g) for x in h.ravel()], dtype=np.float64)
    return out.reshape(h.shape)


def gauss_F(tau, mu_z, sig_z, counts, g) -> float:
    """F(tau) = sum_p n_p E[(X_p - tau)_+^g] with X_p ~ N(mu_z[p], sig_z[p]^2)
    (g an int, or a real g >= 1)."""
    mu_z = np.asarray(mu_z, dtype=np.float64)
    sig_z = np.asarray(sig_z, dtype=np.float64)
    counts = np.asarray(counts, dtype=np.float64)
    pos = sig_z > 0.0
    terms = np.empty_like(mu_z)
    sp = sig_z[pos]
    terms[pos] = sp ** g * partial_moment_real((mu_z[pos] - tau) / sp, g)
    terms[~pos] = np.maximum(mu_z[~pos] - tau, 0.0) ** g
    return math.fsum(counts * terms)


def gauss_tau_hat(mu_z, sig_z, counts, g, max_iter: int = 400) -> float:
    """Root of F(tau) = 1 by bracketing then bisection to fp64 convergence."""
    mu_z = np.asarray(mu_z, dtype=np.float64)
    lo = float(mu_z.max()) - 1.0
    if gauss_F(lo, mu_z, sig_z, counts, g) < 1.0:
        raise AssertionError("bracket violated: F(max mu - 1) < 1")
    step = 1.0
    hi = lo + step
    while gauss_F(hi, mu_z, sig_z, counts, g) >= 1.0:
        step *= 2.0
        hi = lo + step
    for _ in range(max_iter):
        mid = 0.5 * (lo + hi)
        if not (lo < mid < hi):
            break
        if gauss_F(mid, mu_z, sig_z, counts, g) >= 1.0:
            lo = mid
        else:
            hi = mid
    return lo


def gauss_select(u_heads, m_heads, v_heads, counts, alpha: float, delta: float):
    """Gaussian-aware selection for one (row, KV head).

    u_heads: fp32 [G][n] box bounds; m_heads, v_heads: fp64 [G][n] score
    moments; counts: valid tokens per page [n].
    Returns (ascending page list, tau_hat [G]).
    """
    g = selection_gamma(alpha)
    a1 = float(alpha) - 1.0
    u_heads = np.asarray(u_heads, dtype=np.float32)
    G, n = u_heads.shape
    keep = np.zeros(n, dtype=bool)
    taus = np.empty(G)
    for h in range(G):
        mu_z = a1 * np.asarray(m_heads[h], dtype=np.float64)
        sig_z = a1 * np.sqrt(np.asarray(v_heads[h], dtype=np.float64))
        t = gauss_tau_hat(mu_z, sig_z, counts, g)
        taus[h] = t
        keep |= a1 * u_heads[h].astype(np.float64) >= t - float(delta)
    if not keep.any():
        U = u_heads.max(axis=0)
        best = max(range(n), key=lambda p: (float(U[p]), -p))
        return [best], taus
    return [int(p) for p in np.nonzero(keep)[0]], taus


def expected_max_std_normal(n: int) -> float:
    """e_n = E[max of n iid N(0, 1)] = integral of x n phi(x) Phi(x)^(n-1) dx (quadrature)."""
    n = int(n)
    if n < 1:
        raise ValueError("n >= 1")
    if n == 1:
        return 0.0

    def f(x):
        return x * n * math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi) * float(ndtr(x)) ** (n - 1)

    with warnings.catch_warnings():
        warnings.simplefilter("ignore", integrate.IntegrationWarning)
        lo = integrate.quad(f, -40.0, 0.0, epsabs=1e-16, epsrel=2e-14, limit=400)[0]
        hi = integrate.quad(f, 0.0, 40.0, epsabs=1e-16, epsrel=2e-14, limit=400)[0]
    return lo + hi


def gauss_est_select(u_heads, m_heads, v_heads, counts, alpha: float, delta: float):
    """Gaussian selection with the expected-maximum estimate (G-est), one (row, KV head).

    Same arguments and results as gauss_select; page p is kept when
    (alpha-1) * (m + e_{n_p} * sqrt(v)) >= tau_hat - delta for a head of the group.
    """
    g = selection_gamma(alpha)
    a1 = float(alpha) - 1.0
    u_heads = np.asarray(u_heads, dtype=np.float32)
    G, n = u_heads.shape
    e_of = {c: expected_max_std_normal(c) for c in set(int(c) for c in counts)}
    e = np.array([e_of[int(c)] for c in counts])
    keep = np.zeros(n, dtype=bool)
    taus = np.empty(G)
    for h in range(G):
        m = np.asarray(m_heads[h], dtype=np.float64)
        v = np.asarray(v_heads[h], dtype=np.float64)
        t = gauss_tau_hat(a1 * m, a1 * np.sqrt(v), counts, g)
        taus[h] = t
        est = m + e * np.sqrt(v)
        keep |= a1 * est >= t - float(delta)
    if not keep.any():
        U = u_heads.max(axis=0)
        best = max(range(n), key=lambda p: (float(U[p]), -p))
        return [best], taus
    return [int(p) for p in np.nonzero(keep)[0]], taus


def gauss_page_masses(mu_z, sig_z, counts, g, tau: float) -> np.ndarray:
    """M_p = n_p E[(X_p - tau)_+^g], X_p ~ N(mu_z[p], sig_z[p]^2) (zero sig: a point mass)."""
    mu_z = np.asarray(mu_z, dtype=np.float64)
    sig_z = np.asarray(sig_z, dtype=np.float64)
    counts = np.asarray(counts, dtype=np.float64)
    pos = sig_z > 0.0
    terms = np.empty_like(mu_z)
    sp = sig_z[pos]
    terms[pos] = sp ** g * partial_moment_real((mu_z[pos] - tau) / sp, g)
    terms[~pos] = np.maximum(mu_z[~pos] - tau, 0.0) ** g
    return counts * terms


def gauss_mass_select(u_heads, m_heads, v_heads, counts, alpha: float, eps: float):
    """Gaussian selection by expected page mass (G-mass), one (row, KV head).

    Same arguments and results as gauss_select, with eps in place of delta:
    page p is kept when n_p E[(X_{h,p} - tau_hat_h)_+^gamma] >= eps for a head
    h of the group.
    """
    g = selection_gamma(alpha)
    a1 = float(alpha) - 1.0
    u_heads = np.asarray(u_heads, dtype=np.float32)
    G, n = u_heads.shape
    keep = np.zeros(n, dtype=bool)
    taus = np.empty(G)
    for h in range(G):
        mu_z = a1 * np.asarray(m_heads[h], dtype=np.float64)
        sig_z = a1 * np.sqrt(np.asarray(v_heads[h], dtype=np.float64))
        t = gauss_tau_hat(mu_z, sig_z, counts, g)
        taus[h] = t
        keep |= gauss_page_masses(mu_z, sig_z, counts, g, t) >= float(eps)
    if not keep.any():
        U = u_heads.max(axis=0)
        best = max(range(n), key=lambda p: (float(U[p]), -p))
        return [best], taus
    return [int(p) for p in np.nonzero(keep)[0]], taus
