"""Pins of the oracle's whole decode step against the theory of the EntmaxKV page.

§3 "Analyse Théorique": if the kept set contains the support S of the
full-cache entmax distribution, the sparse output equals the full-cache output
(support recovery); in general ||o - o~|| <= 2 B delta, with B a bound on the
value norms and delta the dropped probability mass.  With p~ the entmax
recomputed on the kept set, in fact ||p~ - p||_1 = 2 delta exactly (the kept
weights grow by exactly the mass the dropped tokens lose).
"""
import math

import numpy as np
import pytest
import torch

from oracle import pipeline
from sparse_kv_cache_page_amd import workloads as wl


def _tiny(seed, **kw):
    base = dict(name="t", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=4,
                lens_range=(9, 61), kv_dtype="bf16", q_std=0.6, scale=1.0, alpha=1.5,
                policy="topk", top_k=4, planted_per_kv_head=2, permute_pool=True, seed=seed)
    base.update(kw)
    return wl.Workload(**base)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_support_recovery_brute_force(seed, alpha):
    w = _tiny(seed, alpha=alpha)
    inp = wl.make_inputs(w)
    rng = np.random.default_rng(seed)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            full = pipeline.run_pair(inp, b, g, "dense", with_full=True)
            counts = full["counts"]
            offs = np.concatenate([[0], np.cumsum(counts)])
            # pages holding any support token of any head of the group
            need = set()
            for h in range(w.group):
                for i in np.nonzero(full["p_full"][h] > 0)[0]:
                    need.add(int(np.searchsorted(offs, i, side="right") - 1))
            extra = [p for p in range(len(counts)) if p not in need and rng.random() < 0.3]
            sel = sorted(need | set(extra))
            res = pipeline.run_pair(inp, b, g, "dense", sel_override=sel, with_full=True)
            assert all(res["support_recovered"])
            np.testing.assert_allclose(res["o"], res["o_full"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(res["tau"], res["tau_full"], rtol=0, atol=1e-12)
            assert np.all(res["dropped_mass"] == 0.0)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_error_bound_any_kept_set(seed, alpha):
    w = _tiny(100 + seed, alpha=alpha, planted_per_kv_head=0, q_std=1.5)
    inp = wl.make_inputs(w)
    rng = np.random.default_rng(seed)
    for b in range(w.batch):
        g = int(rng.integers(0, w.num_kv_heads))
        n = len(pipeline.row_pages(inp, b)[0])
        sel = sorted(set(rng.choice(n, size=max(1, n // 2), replace=False).tolist()))
        res = pipeline.run_pair(inp, b, g, "dense", sel_override=sel, with_full=True)
        kept = res["kept_mask"]
        for h in range(w.group):
            d = res["dropped_mass"][h]
            p_sparse = np.zeros(kept.size)
            p_sparse[kept] = res["p"][h]
            l1 = np.abs(p_sparse - res["p_full"][h]).sum()
            assert abs(l1 - 2 * d) <= 1e-12
            err = np.linalg.norm(res["o"][h] - res["o_full"][h])
            assert err <= 2 * res["value_norm_bound"] * d + 1e-12


def test_tiny_config_recovers_planted_support():
    # the tiny decode case: 8 planted keys define the support; top-32 of 256
    # pages by box bound contains them, so sparse == full
    w = wl.CONFIGS["tiny"]
    inp = wl.make_inputs(w)
    res = pipeline.run_pair(inp, 0, 0, "topk", with_full=True)
    assert len(res["sel"]) == 32
    assert all(res["support_recovered"])
    np.testing.assert_allclose(res["o"], res["o_full"], atol=1e-12)
    supp = int((res["p_full"][0] > 0).sum())
    assert 1 <= supp <= 8


def test_padding_never_used():
    # sentinels in padding slots must not reach metadata or outputs
    w = _tiny(7, lens_range=None, seq_len=13, batch=1)
    inp = wl.make_inputs(w)
    res = pipeline.run_pair(inp, 0, 0, "dense")
    assert np.isfinite(res["o"]).all()
    assert max(np.max(np.abs(k)) for k in res["kmax"]) < 100
    assert res["counts"][-1] == 1


def test_widen_bf16_exact():
    x = torch.tensor([1.0, -2.5, 3.140625, 1e-3]).to(torch.bfloat16)
    y = pipeline.widen(x)
    np.testing.assert_array_equal(y, x.float().numpy().astype(np.float64))
