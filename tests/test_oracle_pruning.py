"""The page-pruning rule against the oracle (CPU).

The decode may skip a selected page when, for every head h of the group, its
box bound is below h's z_max - 1 with slack, z_max bounded from below by the
scores of h's best selected page: since no entmax weight exceeds 1, the
threshold satisfies tau >= z_max - 1, so such a page's tokens all get zero
weight (EntmaxKV summary page, §2.C and §3: only the support decides the
output).  Here the rule, written as the library applies it (fp32 bounds and
slacks), is applied to the oracle's own bounds and scores, and every page it
skips must carry zero oracle weight for every head of the group.
"""
import numpy as np
import pytest

from oracle import pipeline
from sparse_kv_cache_page_amd import workloads as wl


def skipped_pages(r, alpha, scale, qq, keys, sel):
    G = qq.shape[0]
    a1 = np.float32(alpha - 1.0)
    u = r["u"]                                     # fp32 [G][n] box bounds
    # z of each selected page's tokens, per head (fp64)
    z = {p: (alpha - 1.0) * scale * (keys[p] @ qq.T) for p in sel}
    zlb = np.empty(G, np.float32)
    for h in range(G):
        best = max(sel, key=lambda p: (float(u[h, p]), -p))
        zlb[h] = np.float32(z[best][:, h].max())
    out = []
    for p in sel:
        x = a1 * u[:, p]
        s1 = np.float32(1e-3) * (np.float32(1) + np.abs(x))
        s2 = np.float32(1e-4) * (np.float32(1) + np.abs(zlb))
        if np.all(x + s1 < zlb - np.float32(1) - s2):
            out.append(p)
    return out


@pytest.mark.parametrize("alpha,seed,planted", [(1.5, 1, 8), (2.0, 2, 8), (1.25, 3, 8),
                                                (1.5, 4, 0), (3.0, 5, 4)])
def test_pruned_pages_carry_no_weight(alpha, seed, planted):
    w = wl.Workload(name="s", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=64,
                    page_size=16, seq_len=3000, kv_dtype="bf16", q_std=0.25, scale=1.0,
                    alpha=alpha, policy="topk", top_k=100, planted_per_kv_head=planted,
                    permute_pool=True, seed=seed)
    inp = wl.make_inputs(w)
    G = w.group
    for g in range(w.num_kv_heads):
        r = pipeline.run_pair(inp, 0, g, "topk")
        sel = list(r["sel"])
        qq = pipeline.widen(inp["q"])[0, g * G:(g + 1) * G]
        _, counts, keys, _ = pipeline.pair_keys_values(inp, 0, g)
        skip = skipped_pages(r, alpha, w.scale, qq, keys, sel)
        # the oracle's weights over the selected tokens, page by page
        offs = np.concatenate([[0], np.cumsum([counts[p] for p in sel])])
        for i, p in enumerate(sel):
            if p in skip:
                assert np.all(r["p"][:, offs[i]:offs[i + 1]] == 0.0), (g, p)
        if planted:
            assert len(skip) > len(sel) // 2, (len(skip), len(sel))
