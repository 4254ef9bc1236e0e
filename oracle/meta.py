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
    as fp32, rounded to nearest from the fp64 value -- or, in the compact
    format, as bf16, rounded once to nearest (ties to an even last bit) from
    the fp64 value.

Pins (tests/test_oracle_meta_scores.py): bounding box by brute force (every key lies
inside, every face is attained); moments of constructed pages with known
closed-form mean and variance; a one-token page has k_min = k_max = k and zero
variance; the bf16 rounding against hand-worked ties and a value that rounding
through fp32 first would get wrong, and on random values against both of its
bf16 neighbours.
"""
from __future__ import annotations

import math

import numpy as np


def round_bf16(x):
    """The bf16 value nearest to each fp64 x (ties to an even last bit), in fp64.

    A bf16 number has 8 significant bits and the exponent range of fp32; below
    2^-126 its spacing stays 2^-133.  With x = m 2^e, 0.5 <= m < 1, the
    spacing at x is 2^(e-8): x / spacing is exact in fp64, rounded half-even
    to an integer, and scaled back exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(np.abs(x))
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.round(x / q) * q                      # numpy rounds halves to even


def store_moments(mean64, var64, moments: str = "f32"):
    """Storage rounding of fp64 moments: 'f32' (nearest fp32) or 'bf16' (round_bf16)."""
    if moments == "bf16":
        return round_bf16(mean64).astype(np.float32), round_bf16(var64).astype(np.float32)
    if moments != "f32":
        raise ValueError(moments)
    return np.asarray(mean64).astype(np.float32), np.asarray(var64).astype(np.float32)


def page_meta(keys, moments: str = "f32"):
    """Metadata of one page from its valid keys.

    keys: array [n][d] (n >= 1) of the exact key values (fp64).
    Returns (kmin, kmax, mean, var): kmin/kmax fp64 holding exact key values,
    mean/var float32 arrays holding the stored values (fp32, or bf16 values
    with moments='bf16').
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
    return (kmin, kmax) + store_moments(mean64, var64, moments)


def page_meta_fast(keys, moments: str = "f32"):
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
    return (kmin, kmax) + store_moments(mu, var, moments)
