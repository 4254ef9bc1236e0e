"""Query-aware page scores from page metadata, in fp64 (oracle; test infrastructure).

EntmaxKV page, §2.A "Notation de Page Consciente de la Requête":
  * Bounding-box bound: from k_min and k_max the scorer gets a deterministic
    upper bound on the largest attention score any token of the page can reach
    for query q.  For one coordinate, q_j k_j is linear in k_j, so over
    k_j in [kmin_j, kmax_j] it peaks at an end point; summing the per-coordinate
    maxima gives
        u = scale * sum_j max(q_j kmin_j, q_j kmax_j)  >=  scale * <q, k>
    for every key k of the page.
  * Gaussian statistics: with per-coordinate mean mu_j and variance sigma2_j of
    the page's keys, the token score scale*<q, k> is modelled as a Gaussian of
    mean  m = scale * sum_j q_j mu_j
    and variance  v = scale^2 * sum_j q_j^2 sigma2_j  (coordinates independent).

Precision: the products q_j * k_j of an fp32 query and bf16/fp32 keys are
exact in fp64; the bound is the correctly rounded sum (math.fsum) times scale,
rounded to nearest fp32.  Ranking uses that fp32 value.

Pins (tests/test_oracle_scores.py): u >= every exact token score by brute force,
u == the score for a one-token page, hand-worked small cases, and the Gaussian
mean/variance against the sample mean/variance of many independent draws.
"""
from __future__ import annotations

import math

import numpy as np


def box_bound(q, kmin, kmax, scale: float) -> np.float32:
    """fp32 upper bound for one (query head, page)."""
    q = np.asarray(q, dtype=np.float64)
    a = q * np.asarray(kmin, dtype=np.float64)
    b = q * np.asarray(kmax, dtype=np.float64)
    terms = np.where(a > b, a, b)
    return np.float32(float(scale) * math.fsum(terms))


def box_bounds(q, kmin, kmax, scale: float) -> np.ndarray:
    """Bounds of many pages for one head: kmin/kmax [npages][d] -> fp32 [npages]."""
    return np.array([box_bound(q, kmin[p], kmax[p], scale) for p in range(len(kmin))],
                    dtype=np.float32)


def gauss_moments(q, mean32, var32, scale: float):
    """(m, v) in fp64 for one (query head, page) from the stored fp32 moments."""
    q = np.asarray(q, dtype=np.float64)
    mu = np.asarray(mean32, dtype=np.float64)
    s2 = np.asarray(var32, dtype=np.float64)
    sc = float(scale)
    m = sc * math.fsum(q * mu)
    v = sc * sc * math.fsum(q * q * s2)
    return m, v
