"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
workload's inputs, then compare one (row, KV head) pair with the CPU oracle.

Tolerances (GPU vs oracle, same input bits):
  kmin/kmax            bit-exact
  mean/var             <= 1 ulp fp32 (both round an fp64 value once)
  u, U                 <= 1 ulp fp32 (fp64 accumulation of exact products,
                        rounded once; the oracle rounds the exact sum)
  sel, n_sel           bit-exact
  gm, gv               <= 1e-12 of the sum of the terms' magnitudes (fp64
                        sums of exact products; v: of v itself)
  tau-hat              <= 1e-12 relative (both fp64; different root finders)
  tau (entmax)         <= 1e-5 absolute, z-space (or 4 fp32 ulps of |tau|
                        when larger: above |tau| ~ 40 fp32 scores cannot
                        resolve 1e-5)
  out                  relative L2 <= 1e-3 per query head
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import pipeline, scores, select
from sparse_kv_cache_page_amd import binding as B

TAU_TOL = 1e-5
TAU_TOL_REL = 4.0 * 2.0 ** -24
OUT_TOL = 1e-3
TAU_HAT_RTOL = 1e-12
MOM_RTOL = 1e-12


def cache_shape(inp) -> B.CacheShape:
    w = inp["workload"]
    return B.CacheShape(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                        inp["max_pages"], inp["num_phys_pages"],
                        torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32,
                        torch.bfloat16 if w.moments_bf16 else torch.float32)


def run_gpu(inp, policy, *, alpha=None, top_k=None, delta=None, scale=None, q=None,
            sel=None, n_sel=None, max_sel=0, prune=True):
    """Whole step on the GPU with every intermediate kept (ub, gm, gv ...).

    With `sel`/`n_sel` given (device int32), selection is skipped and the
    decode runs over that page list.  prune: the decode skips the pages its
    per-head bounds place below every head's support (ub / zlb arguments).
    """
    w = inp["workload"]
    s = cache_shape(inp)
    dev = inp["K"].device
    alpha = w.alpha if alpha is None else alpha
    top_k = w.top_k if top_k is None else top_k
    delta = w.delta if delta is None else delta
    scale = w.scale if scale is None else scale
    q = inp["q"] if q is None else q
    Bt, Hq, Hkv, d, mp, Np = (s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim,
                              s.max_pages_per_seq, s.num_phys_pages)
    o = {}
    o["kmin"] = torch.full((Np, Hkv, d), float("nan"), dtype=s.kv_dtype, device=dev)
    o["kmax"] = torch.full((Np, Hkv, d), float("nan"), dtype=s.kv_dtype, device=dev)
    o["mean"] = torch.full((Np, Hkv, d), float("nan"), dtype=s.moments_dtype, device=dev)
    o["var"] = torch.full((Np, Hkv, d), float("nan"), dtype=s.moments_dtype, device=dev)
    B.build_page_meta(s, inp["K"], inp["block_table"], inp["seq_lens"], o["kmin"], o["kmax"],
                      o["mean"], o["var"])
    o["ub"] = torch.full((Bt, w.num_kv_heads, mp, w.group), float("nan"), dtype=torch.float32,
                         device=dev)
    o["ubg"] = torch.full((Bt, Hkv, mp), float("nan"), dtype=torch.float32, device=dev)
    gauss = policy in ("gauss", "gauss_est", "gauss_mass")
    if gauss:
        o["gm"] = torch.full((Bt, Hq, mp), float("nan"), dtype=torch.float64, device=dev)
        o["gv"] = torch.full((Bt, Hq, mp), float("nan"), dtype=torch.float64, device=dev)
        o["tau_hat"] = torch.full((Bt, Hq), float("nan"), dtype=torch.float64, device=dev)
    B.score_pages(s, q, scale, o["kmin"], o["kmax"], inp["block_table"], inp["seq_lens"],
                  o["ubg"], ub=o["ub"], mean=o["mean"] if gauss else None,
                  var=o["var"] if gauss else None, gm=o.get("gm"), gv=o.get("gv"))
    if sel is None and policy != "dense":
        o["sel"] = torch.full((Bt, Hkv, mp), -7, dtype=torch.int32, device=dev)
        o["n_sel"] = torch.full((Bt, Hkv), -7, dtype=torch.int32, device=dev)
        pol = {"topk": B.EKV_SELECT_TOPK, "gauss": B.EKV_SELECT_GAUSS,
               "gauss_est": B.EKV_SELECT_GAUSS_EST, "gauss_mass": B.EKV_SELECT_GAUSS_MASS}[policy]
        B.select_pages(s, inp["seq_lens"], pol, top_k, alpha, delta, o["ubg"], o["sel"],
                       o["n_sel"], ub=o["ub"] if policy == "gauss" else None, gm=o.get("gm"),
                       gv=o.get("gv"), tau_hat=o.get("tau_hat"))
        max_sel = min(top_k, mp) if policy == "topk" else mp
        use_sel, use_n = o["sel"], o["n_sel"]
    elif sel is not None:
        use_sel, use_n = sel, n_sel
    else:
        use_sel = use_n = None
    o["out"] = torch.full((Bt, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    o["tau"] = torch.full((Bt, Hq), float("nan"), dtype=torch.float32, device=dev)
    o["n_support"] = torch.full((Bt, Hq), -7, dtype=torch.int32, device=dev)
    o["zlb"] = torch.full((Bt, Hq), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(B.decode_workspace_bytes(s, max_sel), dtype=torch.uint8, device=dev)
    B.entmax_decode(s, q, scale, alpha, inp["K"], inp["V"], inp["block_table"],
                    inp["seq_lens"], o["out"], ws, sel=use_sel, n_sel=use_n, max_sel=max_sel,
                    tau=o["tau"], n_support=o["n_support"], ub=o["ub"] if prune else None,
                    zlb=o["zlb"] if prune else None)
    torch.cuda.synchronize()
    return o


def ulp_dist(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.ascontiguousarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


def _np(t):
    return pipeline.widen(t)


def check_pair(inp, gpu, b, g, policy, *, alpha=None, top_k=None, delta=None, scale=None,
               sel_override=None, q=None, check_meta=True):
    """Compare one (row b, KV head g) of the GPU step with the oracle; returns the oracle dict."""
    w = inp["workload"]
    G = w.group
    ref = pipeline.run_pair(inp, b, g, policy, alpha=alpha, top_k=top_k, delta=delta,
                            scale=scale, sel_override=sel_override, q=q)
    phys = ref["phys"]
    n = len(phys)
    idx = torch.tensor(phys, dtype=torch.long, device=gpu["kmin"].device)
    if check_meta:
        kmin = _np(gpu["kmin"][idx, g])
        kmax = _np(gpu["kmax"][idx, g])
        np.testing.assert_array_equal(kmin, np.stack(ref["kmin"]), err_msg=f"kmin b{b} g{g}")
        np.testing.assert_array_equal(kmax, np.stack(ref["kmax"]), err_msg=f"kmax b{b} g{g}")
        if policy in ("gauss", "gauss_est", "gauss_mass"):
            # stored values (fp32, or bf16 values held in fp32): both sides round
            # an fp64 moment once, so they agree to one unit of the storage format
            mu = gpu["mean"][idx, g].float().cpu().numpy()
            va = gpu["var"][idx, g].float().cpu().numpy()
            unit = 1 << 16 if gpu["mean"].dtype == torch.bfloat16 else 1
            assert ulp_dist(mu, np.stack(ref["mean"])).max() <= unit, f"mean b{b} g{g}"
            assert ulp_dist(va, np.stack(ref["var"])).max() <= unit, f"var b{b} g{g}"
    if gpu.get("ub") is not None:   # the fused step keeps them in its workspace
        ub = gpu["ub"][b, g, :n, :].T.cpu().numpy()   # [G][n]
        assert ulp_dist(ub, ref["u"]).max() <= 1, f"u b{b} g{g}"
    ubg = gpu["ubg"][b, g, :n].cpu().numpy()
    assert ulp_dist(ubg, ref["U"]).max() <= 1, f"U b{b} g{g}"
    if policy in ("gauss", "gauss_est", "gauss_mass") and gpu.get("gm") is not None:
        # Gaussian score moments, element by element and stage-wise: the
        # oracle's moment formula is fed the page mean/variance the GPU stored
        # (so a one-ulp difference in a stored moment cannot hide or fake a
        # scoring error).  Both sides sum exact fp64 products (fp32 q times an
        # fp32 or bf16 moment), the oracle correctly rounded, the GPU with at
        # most a dozen fp64 roundings per sum, so they agree to 1e-12 of the
        # sum of the terms' magnitudes (for v, which has no cancellation, that
        # is 1e-12 of v itself)
        gm = gpu["gm"][b, g * G:(g + 1) * G, :n].cpu().numpy()
        gv = gpu["gv"][b, g * G:(g + 1) * G, :n].cpu().numpy()
        sc = float(np.float32(w.scale if scale is None else scale))
        qq = _np(inp["q"] if q is None else q)[b, g * G:(g + 1) * G]      # [G][d]
        mu_g = _np(gpu["mean"][idx, g])                                    # [n][d]
        va_g = _np(gpu["var"][idx, g])
        m_ref = np.empty((G, n))
        v_ref = np.empty((G, n))
        for h in range(G):
            for p in range(n):
                m_ref[h, p], v_ref[h, p] = scores.gauss_moments(qq[h], mu_g[p], va_g[p], sc)
        mag = sc * (np.abs(qq) @ np.abs(mu_g).T)                           # [G][n]
        assert np.all(np.abs(gm - m_ref) <= MOM_RTOL * mag + 1e-300), f"gm b{b} g{g}"
        assert np.all(np.abs(gv - v_ref) <= MOM_RTOL * np.abs(v_ref) + 1e-300), f"gv b{b} g{g}"
    if policy in ("gauss", "gauss_est", "gauss_mass"):
        th = gpu["tau_hat"][b, g * G:(g + 1) * G].cpu().numpy()
        np.testing.assert_allclose(th, ref["tau_hat"], rtol=TAU_HAT_RTOL, atol=1e-300,
                                   err_msg=f"tau_hat b{b} g{g}")
    if sel_override is None and policy != "dense":
        ns = int(gpu["n_sel"][b, g])
        got = gpu["sel"][b, g, :ns].cpu().tolist()
        assert got == list(ref["sel"]), f"sel b{b} g{g}: gpu {got[:12]}.. vs {ref['sel'][:12]}.."
        # stage-wise: the oracle's selection fed the GPU's own bounds (and
        # moments), so a scoring difference cannot mask a selection error
        k_eff = w.top_k if top_k is None else top_k
        if policy == "topk":
            st = select.topk_pages(ubg, k_eff)
            if st != got:
                srt = np.sort(ubg.astype(np.float64))[::-1]
                gap = (srt[k_eff - 1] - srt[k_eff]) / abs(srt[k_eff - 1]) if k_eff < n else None
                raise AssertionError(f"stage-wise top-k b{b} g{g} differs (k-th gap {gap})")
        elif gpu.get("gm") is not None:
            a_ = float(np.float32(w.alpha if alpha is None else alpha))
            d_ = float(np.float32(w.delta if delta is None else delta))
            rule = {"gauss": select.gauss_select, "gauss_est": select.gauss_est_select,
                    "gauss_mass": select.gauss_mass_select}[policy]
            u_g = gpu["ub"][b, g, :n, :].T.cpu().numpy() if gpu.get("ub") is not None else ref["u"]
            st, th_st = rule(u_g, gm, gv, ref["counts"], a_, d_)
            assert st == got, f"stage-wise {policy} b{b} g{g} differs"
            np.testing.assert_allclose(gpu["tau_hat"][b, g * G:(g + 1) * G].cpu().numpy(), th_st,
                                       rtol=TAU_HAT_RTOL, atol=1e-300,
                                       err_msg=f"stage-wise tau_hat b{b} g{g}")
    tau = gpu["tau"][b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
    tol = np.maximum(TAU_TOL, TAU_TOL_REL * np.abs(ref["tau"]))
    assert np.all(np.abs(tau - ref["tau"]) <= tol), \
        f"tau b{b} g{g}: {tau} vs {ref['tau']} (diff {np.abs(tau - ref['tau']).max():.3e})"
    out = gpu["out"][b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
    for h in range(G):
        den = np.linalg.norm(ref["o"][h])
        err = np.linalg.norm(out[h] - ref["o"][h]) / max(den, 1e-30)
        assert err <= OUT_TOL, f"out b{b} g{g} h{h}: rel L2 {err:.3e}"
    return ref
