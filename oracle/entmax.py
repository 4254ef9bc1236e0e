"""alpha-entmax over a vector of scores, in fp64 (oracle; test infrastructure).

The EntmaxKV page (§2 "Méthodologie") states that alpha-entmax with alpha > 1
yields probability vectors with exact zeros, and (§2.B) that the method works
with the global entmax threshold tau.  The mapping itself is the standard one:

    p_i = [ z_i - tau ]_+ ^ (1/(alpha-1)),   z_i = (alpha-1) * s_i,

with tau the unique value for which sum_i p_i = 1.  tau is always expressed in
the z-space above.

Bracket used for the root (derived from the definition):
  * the largest weight is at most 1, so tau >= z_max - 1;
  * n weights each at most (z_max - tau)^gamma sum to 1, so
    tau <= z_max - n^(1-alpha).
f(tau) = sum_i [z_i - tau]_+^gamma - 1 is continuous and strictly decreasing
where positive, so plain bisection on that bracket converges to tau.

Pins (tests/test_oracle_entmax.py): alpha = 2 against the sort-based sparsemax
closed form, alpha = 1.5 against the quadratic closed form per support size,
alpha -> 1 against softmax, sum = 1, exact zeros, bracket, hand-worked cases.
"""
from __future__ import annotations

import math

import numpy as np


def gamma_of(alpha: float) -> float:
    """Exponent 1/(alpha-1) of the entmax weights; alpha must exceed 1."""
    if not (alpha > 1.0):
        raise ValueError("alpha-entmax needs alpha > 1")
    return 1.0 / (float(alpha) - 1.0)


def _power(x: np.ndarray, gamma: float) -> np.ndarray:
    # x >= 0 elementwise; integer exponents are evaluated by repeated product so
    # that the common cases (gamma = 1, 2, 4) are free of pow() rounding.
    if float(gamma).is_integer():
        out = np.ones_like(x)
        for _ in range(int(gamma)):
            out = out * x
        return out
    return np.power(x, gamma)


def threshold(z, alpha: float, max_iter: int = 400) -> float:
    """tau with sum_i [z_i - tau]_+^gamma = 1, by bisection in fp64.

    `z` holds the z-space scores (alpha-1)*s of one query head over the tokens
    it may attend to; entries equal to -inf are absent tokens.
    """
    z = np.asarray(z, dtype=np.float64)
    z = z[np.isfinite(z)]
    n = z.size
    if n == 0:
        raise ValueError("entmax over an empty token set is undefined")
    gamma = gamma_of(alpha)
    zmax = float(z.max())
    lo = zmax - 1.0
    hi = zmax - float(n) ** (1.0 - float(alpha))
    if hi < lo:          # n == 1 gives hi == lo exactly
        hi = lo
    for _ in range(max_iter):
        mid = 0.5 * (lo + hi)
        if not (lo < mid < hi):
            break
        f = math.fsum(_power(np.maximum(z - mid, 0.0), gamma)) - 1.0
        if f >= 0.0:
            lo = mid
        else:
            hi = mid
    # lo and hi are now adjacent doubles (or equal); either brackets the root
    return lo


def weights(z, tau: float, alpha: float) -> np.ndarray:
    """p_i = [z_i - tau]_+^gamma (exact zeros off the support)."""
    z = np.asarray(z, dtype=np.float64)
    d = np.where(np.isfinite(z), z - tau, -1.0)
    return _power(np.maximum(d, 0.0), gamma_of(alpha))


def entmax_scores(s, alpha: float):
    """(tau, p) for raw scores s (z = (alpha-1) s)."""
    s = np.asarray(s, dtype=np.float64)
    z = (float(alpha) - 1.0) * s
    tau = threshold(z, alpha)
    return tau, weights(z, tau, alpha)


def softmax(s) -> np.ndarray:
    """The alpha = 1 member of the family (dense); used only to pin alpha -> 1."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / math.fsum(e)
