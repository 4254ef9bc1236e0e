"""Softmax decode over a kept token set, in fp64 (oracle; test infrastructure).

The EntmaxKV page contrasts its method with sparse decoding under softmax
(§1, §3 "Analyse Théorique", §4 "Résultats"): softmax gives every token a
strictly positive weight, so dropping any token drops mass delta > 0 and the
output error is only bounded (||o - o~|| <= 2 B delta), whereas alpha-entmax
drops nothing once the kept set holds its support.  Its speed comparison is
against a full-cache softmax decode (FlashDecoding, §4).  This module gives
the softmax side of that comparison:

    s_i = scale * <q, k_i>,   lse = log sum_i exp(s_i),
    p_i = exp(s_i - lse),     o = sum_i p_i v_i

over the valid tokens of the kept pages (all pages for the full cache).
The dropped softmax mass of a kept set I is delta = 1 - exp(lse_I - lse_all),
and renormalising the kept weights moves exactly 2 delta of L1 mass, so
||o_I - o_all|| <= 2 B delta with B the largest value-row norm.

Pins (tests/test_oracle_softmax.py): one token gives o = v and lse = s;
equal scores give the plain mean of the values and lse = s + log n; the
alpha -> 1 limit of the entmax oracle; a shift of every score moves lse by
the shift and leaves o unchanged; the 2 delta identity and 2 B delta bound
on random kept sets; brute-force two-token values.
"""
from __future__ import annotations

import math

import numpy as np


def softmax_decode_heads(q_heads, keys, vals, scale: float):
    """Softmax attention of each head over the given tokens.

    q_heads [G][d]; keys/vals [n][d] (n >= 1).  Returns (lse [G], p [G][n], o [G][d]),
    with lse the natural log of sum_i exp(scale <q_h, k_i>).
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    lses, ps, outs = [], [], []
    for h in range(q_heads.shape[0]):
        s = float(scale) * (keys @ q_heads[h])
        m = float(s.max())
        e = np.exp(s - m)
        lse = m + math.log(math.fsum(e))
        p = np.exp(s - lse)
        lses.append(lse)
        ps.append(p)
        outs.append(p @ vals)
    return np.array(lses), np.array(ps), np.array(outs)


def dropped_mass(lse_kept, lse_all):
    """Softmax mass of the tokens outside the kept set: 1 - exp(lse_kept - lse_all)."""
    return 1.0 - np.exp(np.asarray(lse_kept, dtype=np.float64) -
                        np.asarray(lse_all, dtype=np.float64))
