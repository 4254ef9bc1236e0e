"""Per-page key metadata, in fp64 (oracle; test infrastructure).

The EntmaxKV page (§2.A "Notation de Page Consciente de la Requête") keeps,
for every page of the paged KV cache, lightweight metadata read before any
key or value:
  * the per-coordinate bounding box of the page's keys, k_min and k_max;
  * the first and second moments of the page's keys (mean and variance), from
    which token scores inside the page are modelled as Gaussian.

Readings taken where the page is silent:
  * moments are per coordinate (diagonal), the variance is the population
    variance (divide by n), over the page's valid tokens only;
  * k_min/k_max are exact (same dtype as the keys), mean/variance are stored
    as fp32, rounded to nearest from the fp64 value.

Pins (tests/test_oracle_meta.py): bounding box by brute force (every key lies
inside, every face is attained); moments of constructed pages with known
closed-form mean and variance; a one-token page has k_min = k_max = k and zero
variance.
"""
from __future__ import annotations

import math

import numpy as np


def page_meta(keys):
    """Metadata of one page from its valid keys.

    keys: array [n][d] (n >= 1) of the exact key values (fp64).
    Returns (kmin, kmax, mean32, var32): kmin/kmax fp64 holding exact key
    values, mean32/var32 float32 arrays.
    """
    k = np.asarray(keys, dtype=np.float64)
    n, d = k.shape
    if n < 1:
        raise ValueError("a page needs at least one valid token")
    kmin = np.empty(d)
    kmax = np.empty(d)
    mean64 = np.empty(d)
    var64 = np.empty(d)
    for j in range(d):
        col = k[:, j]
        lo = col[0]
        hi = col[0]
        for x in col[1:]:
            if x < lo:
                lo = x
            if x > hi:
                hi = x
        kmin[j] = lo
        kmax[j] = hi
        mu = math.fsum(col) / n
        mean64[j] = mu
        var64[j] = math.fsum((col - mu) ** 2) / n
    return kmin, kmax, mean64.astype(np.float32), var64.astype(np.float32)


def page_meta_fast(keys):
    """Same quantities as page_meta, vectorised over pages.

    keys: [npages][n][d] with the same n valid tokens in every page.  Uses
    numpy reductions (pairwise fp64 sums) in place of fsum; the two agree to
    fp64 rounding, far below the fp32 storage precision.  Used for large
    cases; page_meta is the reference it is checked against.
    """
    k = np.asarray(keys, dtype=np.float64)
    n = k.shape[1]
    kmin = k.min(axis=1)
    kmax = k.max(axis=1)
    mu = k.sum(axis=1) / n
    var = ((k - mu[:, None, :]) ** 2).sum(axis=1) / n
    return kmin, kmax, mu.astype(np.float32), var.astype(np.float32)
