"""The whole decode step for one (row b, KV head g), in fp64 (oracle; test infrastructure).

EntmaxKV page, §2 "Méthodologie": a paged decode pipeline of three parts --
query-aware page scoring from per-page metadata (§2.A), a candidate selection
policy (§2.B), and alpha-entmax attention over the keys and values of the
selected pages only (§2.C).  §3 "Analyse Théorique": if the kept set contains
the support of the full-cache entmax distribution, the sparse output equals
the full-cache output; otherwise ||o - o~|| <= 2 B delta.

Inputs are read back bit-exactly from the tensors the workload generator drew
(bf16 through its bit pattern), so the oracle sees what the GPU sees.
"""
from __future__ import annotations

import numpy as np

from . import entmax, meta, scores, select


def widen(t) -> np.ndarray:
    """Exact fp64 copy of a torch fp32/bf16/int tensor (bf16 via its bits)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.cpu().contiguous().view(torch.int16).numpy().astype(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if t.dtype in (torch.int32, torch.int64):
        return t.cpu().numpy()
    return t.cpu().numpy().astype(np.float64)


def row_pages(inputs: dict, b: int):
    """(physical page ids, valid-token counts) of row b in logical order."""
    P = inputs["workload"].page_size
    L = int(inputs["lens"][b])
    n = (L + P - 1) // P
    phys = [int(x) for x in inputs["block_table"][b, :n].cpu().tolist()]
    counts = [P] * (n - 1) + [L - (n - 1) * P]
    return phys, counts


def pair_keys_values(inputs: dict, b: int, g: int):
    """Exact fp64 keys and values of row b, KV head g: lists of [n_p][d] arrays per page."""
    import torch
    phys, counts = row_pages(inputs, b)
    idx = torch.tensor(phys, dtype=torch.long, device=inputs["K"].device)
    Kt = widen(inputs["K"][idx, g])      # [n][P][d]
    Vt = widen(inputs["V"][idx, g])
    keys = [Kt[i, : counts[i]] for i in range(len(phys))]
    vals = [Vt[i, : counts[i]] for i in range(len(phys))]
    return phys, counts, keys, vals


def pair_meta(keys, exact: bool = False, moments: str = "f32"):
    """Metadata of every page of a pair (lists of kmin, kmax, mean, var)."""
    if exact:
        out = [meta.page_meta(k, moments) for k in keys]
        return ([o[0] for o in out], [o[1] for o in out],
                [o[2] for o in out], [o[3] for o in out])
    n_full = [i for i, k in enumerate(keys) if k.shape[0] == keys[0].shape[0]]
    res = [None] * len(keys)
    if n_full:
        kmin, kmax, mu, var = meta.page_meta_fast(np.stack([keys[i] for i in n_full]), moments)
        for j, i in enumerate(n_full):
            res[i] = (kmin[j], kmax[j], mu[j], var[j])
    for i, k in enumerate(keys):
        if res[i] is None:
            res[i] = meta.page_meta(k, moments)
    return ([r[0] for r in res], [r[1] for r in res], [r[2] for r in res], [r[3] for r in res])


def decode_heads(q_heads, keys_sel, vals_sel, scale: float, alpha: float):
    """alpha-entmax attention of each head over the given tokens.

    q_heads [G][d]; keys_sel/vals_sel [n][d].  Returns (tau [G], p [G][n], o [G][d]).
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    a1 = float(alpha) - 1.0
    taus, ps, outs = [], [], []
    for h in range(q_heads.shape[0]):
        s = float(scale) * (keys_sel @ q_heads[h])
        z = a1 * s
        tau = entmax.threshold(z, alpha)
        p = entmax.weights(z, tau, alpha)
        taus.append(tau)
        ps.append(p)
        outs.append(p @ vals_sel)
    return np.array(taus), np.array(ps), np.array(outs)


def run_pair(inputs: dict, b: int, g: int, policy: str, *, alpha=None, top_k=None,
             delta=None, scale=None, q=None, exact_meta=False, with_full=False,
             sel_override=None, timings=None):
    """One decode step of (row b, KV head g) under `policy` ('topk', 'gauss', 'gauss_est',
    'gauss_mass', 'dense').

    alpha, scale and delta are the fp32 values handed to the library (widened).
    Returns a dict with the metadata, bounds, selection and entmax outputs.
    If `timings` is a dict, wall-clock seconds of the phases are added to it
    under 'read', 'meta', 'score', 'select' and 'decode'.
    """
    import time
    clock = [time.perf_counter()]

    def lap(name):
        if timings is not None:
            now = time.perf_counter()
            timings[name] = timings.get(name, 0.0) + now - clock[0]
            clock[0] = now

    w = inputs["workload"]
    alpha = float(np.float32(w.alpha if alpha is None else alpha))
    scale = float(np.float32(w.scale if scale is None else scale))
    delta = float(np.float32(w.delta if delta is None else delta))
    top_k = w.top_k if top_k is None else top_k
    G = w.group
    qq = widen(inputs["q"] if q is None else q)[b, g * G:(g + 1) * G]   # [G][d]

    phys, counts, keys, vals = pair_keys_values(inputs, b, g)
    n = len(phys)
    lap("read")
    kmin, kmax, mu, var = pair_meta(keys, exact=exact_meta,
                                    moments="bf16" if w.moments_bf16 else "f32")
    lap("meta")

    u = np.array([scores.box_bounds(qq[h], kmin, kmax, scale) for h in range(G)],
                 dtype=np.float32)                                     # [G][n]
    U = u.max(axis=0)
    out = dict(phys=phys, counts=counts, kmin=kmin, kmax=kmax, mean=mu, var=var,
               u=u, U=U, tau_hat=None)

    lap("score")
    if sel_override is not None:
        sel = list(sel_override)
    elif policy == "topk":
        sel = select.topk_pages(U, top_k)
    elif policy == "dense":
        sel = list(range(n))
    elif policy in ("gauss", "gauss_est", "gauss_mass"):
        m = np.empty((G, n))
        v = np.empty((G, n))
        for h in range(G):
            for p in range(n):
                m[h, p], v[h, p] = scores.gauss_moments(qq[h], mu[p], var[p], scale)
        rule = {"gauss": select.gauss_select, "gauss_est": select.gauss_est_select,
                "gauss_mass": select.gauss_mass_select}[policy]
        # delta: the margin of the maximum-score rules, the mass threshold of G-mass
        sel, tau_hat = rule(u, m, v, counts, alpha, delta)
        out.update(m=m, v=v, tau_hat=tau_hat)
    else:
        raise ValueError(policy)
    out["sel"] = sel
    lap("select")

    ks = np.concatenate([keys[p] for p in sel])
    vs = np.concatenate([vals[p] for p in sel])
    tau, p, o = decode_heads(qq, ks, vs, scale, alpha)
    out.update(tau=tau, p=p, o=o, n_tokens=ks.shape[0])
    lap("decode")

    if with_full:
        kf = np.concatenate(keys)
        vf = np.concatenate(vals)
        tau_f, p_f, o_f = decode_heads(qq, kf, vf, scale, alpha)
        # token offsets of each page inside the full concatenation
        offs = np.concatenate([[0], np.cumsum(counts)])
        kept = np.zeros(kf.shape[0], dtype=bool)
        for pg in sel:
            kept[offs[pg]:offs[pg + 1]] = True
        delta_mass = p_f[:, ~kept].sum(axis=1)
        support_in = [(p_f[h] > 0)[~kept].sum() == 0 for h in range(G)]
        B = np.sqrt((vf * vf).sum(axis=1)).max()
        out.update(tau_full=tau_f, p_full=p_f, o_full=o_f, dropped_mass=delta_mass,
                   support_recovered=support_in, value_norm_bound=B, kept_mask=kept)
    return out


def softmax_pair(inputs: dict, b: int, g: int, sel, *, scale=None, q=None):
    """Softmax decode of (row b, KV head g) over the pages `sel` (None: every page),
    and over the full cache: the comparison of §3-§4 of the EntmaxKV page.

    Returns dict(lse, o) of the kept set, (lse_full, o_full), the dropped softmax
    mass delta per head and the largest value-row norm B of the row.
    """
    from . import softmax
    w = inputs["workload"]
    scale = float(np.float32(w.scale if scale is None else scale))
    G = w.group
    qq = widen(inputs["q"] if q is None else q)[b, g * G:(g + 1) * G]
    phys, counts, keys, vals = pair_keys_values(inputs, b, g)
    kf = np.concatenate(keys)
    vf = np.concatenate(vals)
    lse_f, _, o_f = softmax.softmax_decode_heads(qq, kf, vf, scale)
    if sel is None:
        sel = list(range(len(phys)))
    ks = np.concatenate([keys[p] for p in sel])
    vs = np.concatenate([vals[p] for p in sel])
    lse, _, o = softmax.softmax_decode_heads(qq, ks, vs, scale)
    return dict(lse=lse, o=o, lse_full=lse_f, o_full=o_f,
                dropped_mass=softmax.dropped_mass(lse, lse_f),
                value_norm_bound=np.sqrt((vf * vf).sum(axis=1)).max())
