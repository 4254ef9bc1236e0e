#!/usr/bin/env python3
"""Decode-step benchmark of the paged alpha-entmax decode library on one GPU.

One step = one decode step of one attention layer for every sequence and query
head of the batch:
    score_pages -> select_pages -> entmax_decode
(top-k policy: the fused score_select_pages, then entmax_decode).  Page
metadata is built before timing; the per-step rebuild of each row's last page
(build_page_meta with first_page = last page, span = 1) is timed on its own and
reported next to the step.  Inputs (K/V pages, metadata, queries) are resident
in HBM before timing.  R
independent layers (own K, V, metadata, queries) are cycled so that the bytes
touched between two visits of a layer exceed the 256 MB Infinity Cache.

Prints one JSON line: steps/s (value), effective KV GB/s and its fraction of
the 8 TB/s HBM peak, the roofline of the dominant entry point, and the CPU
oracle timed on a bounded sample of the same step.

    python bench.py [--steps K] [--warmup W] [--config gqa] [--layers R]
                    [--no-graph] [--cpu-seconds S] [--no-sweep] [--no-comparison]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")
# sources whose change invalidates recorded HBM counters, per entry point
KERNEL_SOURCES = {  # the HIP file of each entry point; local includes are followed
    "ekv_score_select_pages": "score.hip",
    "ekv_entmax_decode": "decode.hip",
    "ekv_score_pages": "score.hip",
    "ekv_select_pages": "select.hip",
    "ekv_build_page_meta": "meta.hip",
    "ekv_append_token": "meta.hip",
    "ekv_topk_decode": "step.hip",
    "ekv_score_box_pages": "score.hip",
}
ENTRY_POINT = {"refresh": "ekv_build_page_meta", "score": "ekv_score_pages",
               "select": "ekv_select_pages", "decode": "ekv_entmax_decode",
               "score_select": "ekv_score_select_pages", "append": "ekv_append_token",
               "topk_decode": "ekv_topk_decode", "score_box": "ekv_score_box_pages"}
METRIC = "decode steps/s + effective KV GB/s (fraction of HBM peak), batch×ctx sweep"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="gqa",
                    help="tiny | gqa | gauss | gauss_est | gauss_mass | ragged | stress")
    ap.add_argument("--layers", type=int, default=0, help="layers cycled (0 = auto)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle sample budget (0 disables the cpu_baseline leg)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the batch x ctx sweep that the gqa run reports with its line")
    ap.add_argument("--no-comparison", action="store_true",
                    help="skip the softmax / full-cache comparison of the gqa run")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the ragged and stress workloads the gqa run reports with its line")
    ap.add_argument("--comparison", action="store_true",
                    help="also run the softmax / full-cache comparison on a top-k workload "
                         "other than gqa")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--policy", default=None)
    ap.add_argument("--top-k", type=int, default=None)
    ap.add_argument("--temperature", type=float, default=None,
                    help="query std * sqrt(d) (stress workload)")
    ap.add_argument("--counter-summary", default="", metavar="CSV",
                    help="only summarise a rocprofv3 --pmc counter_collection.csv per kernel "
                         "(dispatches, mean counter value, mean duration) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for "
                         "HBM byte counters) and exit")
    return ap.parse_args()


class Layer:
    """One attention layer's cache, queries and decoder buffers."""

    def __init__(self, w, seed_offset, dev):
        import torch
        from sparse_kv_cache_page_amd import workloads as wl
        from sparse_kv_cache_page_amd.binding import CacheShape
        from sparse_kv_cache_page_amd.engine import PagedEntmaxDecoder
        self.w = wl.variant(w, seed=w.seed + seed_offset)
        self.inp = wl.make_inputs(self.w, device=dev)
        inp = self.inp
        self.shape = CacheShape(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                inp["max_pages"], inp["num_phys_pages"],
                                torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32,
                                torch.bfloat16 if w.moments_bf16 else torch.float32)
        self.dec = PagedEntmaxDecoder(self.shape, policy=w.policy, top_k=w.top_k,
                                      alpha=w.alpha, scale=w.scale, delta=w.delta, device=dev,
                                      fused=w.policy == "topk")
        self.dec.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
        self.last_page = torch.tensor([n - 1 for n in inp["npages"]], dtype=torch.int32,
                                      device=dev)
        # each row's last token, re-appended by the timed append (idempotent)
        rows = torch.arange(w.batch, device=dev)
        t = (inp["seq_lens"] - 1).long()
        pi = inp["block_table"][rows, t // w.page_size].long()
        self.k_last = inp["K"][pi, :, t % w.page_size].contiguous()
        self.v_last = inp["V"][pi, :, t % w.page_size].contiguous()

    # the calls of one step, separately so they can be timed one by one
    @property
    def stages(self):
        if self.w.policy == "topk":
            return ["score_box", "topk_decode"]
        if self.w.policy == "dense":
            return ["decode"]
        return ["score", "select", "decode"]

    def score_select(self):
        i = self.inp
        self.dec.score_select(i["q"], i["K"], i["block_table"], i["seq_lens"])

    def refresh(self):
        i = self.inp
        self.dec.build_meta(i["K"], i["block_table"], i["seq_lens"], first_page=self.last_page,
                            span=1)

    def append(self):
        i = self.inp
        self.dec.append(self.k_last, self.v_last, i["K"], i["V"], i["block_table"],
                        i["seq_lens"])

    def score(self):
        i = self.inp
        self.dec.score(i["q"], i["block_table"], i["seq_lens"])

    def select(self):
        self.dec.select(self.inp["seq_lens"])

    def decode(self):
        i = self.inp
        self.dec.decode(i["q"], i["K"], i["V"], i["block_table"], i["seq_lens"])

    def score_box(self):
        i = self.inp
        self.dec.score_box(i["q"], i["block_table"], i["seq_lens"])

    def topk_decode(self):
        i = self.inp
        self.dec.topk_decode(i["q"], i["K"], i["V"], i["block_table"], i["seq_lens"],
                             use_hint=True)

    def step(self):
        for n in self.stages:
            getattr(self, n)()

    # the comparison of §3-§4 of the EntmaxKV page: softmax decode over the
    # step's selected pages and over the full cache, and the full-cache entmax
    # decode (buffers made on first use)
    def _cmp_buffers(self):
        if hasattr(self, "cmp"):
            return self.cmp
        import torch
        from sparse_kv_cache_page_amd import binding as Bd
        s, dev = self.shape, self.inp["K"].device
        B, Hq, d = s.batch, s.num_q_heads, s.head_dim
        c = {"o_sm_sel": torch.empty(B, Hq, d, device=dev),
             "o_sm_full": torch.empty(B, Hq, d, device=dev),
             "o_ent_full": torch.empty(B, Hq, d, device=dev),
             "lse_sel": torch.empty(B, Hq, device=dev),
             "lse_full": torch.empty(B, Hq, device=dev),
             "ws_sm_sel": torch.empty(Bd.softmax_workspace_bytes(s, self.dec.max_sel),
                                      dtype=torch.uint8, device=dev),
             "ws_sm_full": torch.empty(Bd.softmax_workspace_bytes(s, 0), dtype=torch.uint8,
                                       device=dev),
             "ws_ent_full": torch.empty(Bd.decode_workspace_bytes(s, 0), dtype=torch.uint8,
                                        device=dev)}
        self.cmp = c
        return c

    def softmax_sel(self):
        from sparse_kv_cache_page_amd import binding as Bd
        c, i = self._cmp_buffers(), self.inp
        Bd.softmax_decode(self.shape, i["q"], self.w.scale, i["K"], i["V"], i["block_table"],
                          i["seq_lens"], c["o_sm_sel"], c["ws_sm_sel"], sel=self.dec.sel,
                          n_sel=self.dec.n_sel, max_sel=self.dec.max_sel, lse=c["lse_sel"])

    def softmax_full(self):
        from sparse_kv_cache_page_amd import binding as Bd
        c, i = self._cmp_buffers(), self.inp
        Bd.softmax_decode(self.shape, i["q"], self.w.scale, i["K"], i["V"], i["block_table"],
                          i["seq_lens"], c["o_sm_full"], c["ws_sm_full"], lse=c["lse_full"])

    def entmax_full(self):
        from sparse_kv_cache_page_amd import binding as Bd
        c, i = self._cmp_buffers(), self.inp
        Bd.entmax_decode(self.shape, i["q"], self.w.scale, self.w.alpha, i["K"], i["V"],
                         i["block_table"], i["seq_lens"], c["o_ent_full"], c["ws_ent_full"])


def stage_bytes(layer):
    """Algorithmic bytes per launch of each entry point (the method's own traffic).

    refresh: valid K rows of each row's last page + the rewritten metadata;
    score:   bounding boxes (+ mean/var for the Gaussian policy) of every page,
             plus the bound written per page;
    select:  bounds read + page lists written;
    decode:  K rows of the selected pages' valid tokens, plus the value rows of
             each head's support (the only value rows entmax needs).
    """
    import torch
    w, inp, dec = layer.w, layer.inp, layer.dec
    e = 2 if w.kv_dtype == "bf16" else 4
    d, P, Hkv = w.head_dim, w.page_size, w.num_kv_heads
    gauss = w.policy in ("gauss", "gauss_est", "gauss_mass")
    lens = inp["lens"]
    npg = inp["npages"]
    last_valid = [L - (n - 1) * P for L, n in zip(lens, npg)]
    mom_e = 2 if w.moments_bf16 else 4          # bytes per stored mean / variance value
    meta_pp = 2 * d * e + (2 * d * mom_e if gauss else 0)
    refresh = sum(Hkv * (v * d * e + meta_pp) for v in last_valid)
    pages = sum(npg) * Hkv
    # per query head: ub (the box-bound Gaussian reading, and the per-head
    # bounds the pruned top-k decode reads) and the fp64 moments
    ub_pp = 4 * w.group if (w.policy == "gauss" or getattr(dec, "prune", False)) else 0
    score = pages * (meta_pp + 4 + ub_pp + (w.group * 16 if gauss else 0))
    if w.policy == "dense":
        n_sel = torch.tensor(npg)[:, None].expand(w.batch, Hkv)
    else:
        n_sel = dec.n_sel.cpu().long()
    select = pages * 4 + int(n_sel.sum()) * 4
    # K rows the decode reads: the valid tokens of every selected page it does
    # not prune (every page is full except a row's last)
    read = page_read_mask(layer)  # [B][Hkv][maxP] over selection slots, or None
    sel = None if w.policy == "dense" else dec.sel.cpu()
    ktok = 0
    for b in range(w.batch):
        for g in range(Hkv):
            ns = int(n_sel[b, g])
            for j in range(ns):
                if read is not None and not read[b, g, j]:
                    continue
                page = j if sel is None else int(sel[b, g, j])
                ktok += last_valid[b] if page == npg[b] - 1 else P
    vrows = int(dec.n_support.cpu().long().sum())
    decode = ktok * d * e + vrows * d * e
    if read is not None:
        # the probe's page per query head, and the bounds of the selected pages
        decode += w.batch * w.num_q_heads * P * d * e + int(n_sel.sum()) * w.group * 4
    full = sum(lens) * Hkv * d * e * 2
    # append: the new K and V rows read and written, the page's box read and
    # written (box-only metadata), or its valid rows read and box + moments
    # written (Gaussian metadata)
    if gauss:
        append = sum(Hkv * (4 * d * e + v * d * e + meta_pp) for v in last_valid)
    else:
        append = w.batch * Hkv * (4 * d * e + 2 * 2 * d * e)
    return dict(refresh=refresh, append=append, score=score if w.policy != "dense" else 0,
                select=select if w.policy != "dense" else 0, decode=decode,
                score_select=score + select, topk_decode=select + decode, score_box=score,
                kv_bytes=(pages * meta_pp if w.policy != "dense" else 0) + decode,
                full_cache=full, k_tokens=ktok, v_rows=vrows)


def page_read_mask(layer):
    """Which selection slots the pruned decode reads (its rule, replayed in fp32)."""
    import torch
    w, dec = layer.w, layer.dec
    if not getattr(dec, "prune", False) or dec.zlb is None:
        return None
    B_, Hkv, G = w.batch, w.num_kv_heads, w.group
    mp = dec.ub.shape[2]
    a1 = torch.tensor(w.alpha - 1.0, dtype=torch.float32)
    ub = dec.ub.cpu().permute(0, 1, 3, 2).contiguous()   # [B][Hkv][G][maxP]
    zlb = dec.zlb.cpu().view(B_, Hkv, G, 1)
    if w.policy == "dense":
        idx = torch.arange(mp).view(1, 1, 1, mp).expand(B_, Hkv, G, mp)
    else:
        idx = dec.sel.cpu().long().clamp(0, mp - 1).view(B_, Hkv, 1, mp).expand(B_, Hkv, G, mp)
    x = a1 * torch.gather(ub, 3, idx)
    s1 = 1e-3 * (1.0 + x.abs())
    s2 = 1e-4 * (1.0 + zlb.abs())
    below = (x + s1 < zlb - 1.0 - s2).all(dim=2)
    return (~below).numpy()


def diagnostics(layer):
    """Diagnostics of one step on one layer (reported, never compared): pages
    selected per (row, KV head), support sizes, how many heads have their
    full-cache entmax support inside the kept pages (the sparse output then
    equals the full-cache one, §3 of the EntmaxKV page), and the entmax mass
    the selection drops, delta = 1 - sum over kept tokens of
    [z - tau_full]_+^gamma with tau_full from the library's full-cache decode.

    The full-cache decode and the step run in the library; the kept-token sum
    for delta is formed here with torch (fp32 scores of the gathered kept keys,
    fp64 sum), which is diagnostics only and not part of the step."""
    import torch
    from sparse_kv_cache_page_amd import binding as Bd
    w, inp, dec, s = layer.w, layer.inp, layer.dec, layer.shape
    layer.step()
    torch.cuda.synchronize()
    Bt, Hq, Hkv, d, G, P = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, w.group, w.page_size
    npg = torch.tensor(inp["npages"], device=inp["K"].device)
    if w.policy == "dense":
        n_sel = npg[:, None].expand(Bt, Hkv)
    else:
        n_sel = dec.n_sel.long()
    out_s, tau_s, sup_s = dec.out.clone(), dec.tau.clone(), dec.n_support.clone()
    out_f = torch.empty_like(out_s)
    tau_f = torch.empty_like(tau_s)
    sup_f = torch.empty_like(sup_s)
    ws = torch.empty(Bd.decode_workspace_bytes(s, 0), dtype=torch.uint8, device=out_s.device)
    Bd.entmax_decode(s, inp["q"], w.scale, w.alpha, inp["K"], inp["V"], inp["block_table"],
                     inp["seq_lens"], out_f, ws, tau=tau_f, n_support=sup_f)
    torch.cuda.synchronize()
    rel = (out_s - out_f).norm(dim=-1) / out_f.norm(dim=-1).clamp_min(1e-30)
    res = {"n_sel": {"mean": float(n_sel.float().mean()), "max": int(n_sel.max())},
           "pages": {"mean": float(npg.float().mean()), "max": int(npg.max())},
           "support_tokens": {"mean": float(sup_f.float().mean()), "max": int(sup_f.max())},
           "heads": int(rel.numel()),
           "sparse_vs_full_output_rel_err": {"median": float(rel.median()),
                                             "max": float(rel.max())}}
    if w.policy == "dense":
        res["entmax_dropped_mass"] = {"mean": 0.0, "max": 0.0, "note": "nothing dropped"}
        res["support_recovery_rate"] = 1.0
        return res
    # kept mass under tau_full, per (row, query head)
    gamma = 1.0 / (w.alpha - 1.0)
    zs = float(w.alpha - 1.0) * float(w.scale)
    mx = int(n_sel.max())
    sel = dec.sel[:, :, :mx].long().clamp(min=0)                        # [B][Hkv][mx]
    live = torch.arange(mx, device=sel.device)[None, None, :] < n_sel[:, :, None]
    page = torch.where(live, sel, torch.zeros_like(sel))
    phys = torch.gather(inp["block_table"].long()[:, None, :].expand(Bt, Hkv, -1), 2, page)
    kept = torch.zeros(Bt, Hq, dtype=torch.float64, device=sel.device)
    for g in range(Hkv):
        kt = inp["K"][phys[:, g], g].float()                              # [B][mx][P][d]
        qh = inp["q"][:, g * G:(g + 1) * G].float()                       # [B][G][d]
        z = zs * torch.matmul(kt.reshape(Bt, mx * P, d), qh.transpose(1, 2).contiguous())
        tok = torch.arange(P, device=sel.device)
        last = page == (npg[:, None, None] - 1)
        nvalid = torch.where(last, (torch.tensor(inp["lens"], device=sel.device)[:, None, None]
                                    - (npg[:, None, None] - 1) * P).expand_as(page),
                             torch.full_like(page, P))
        ok = (live[:, g, :, None] & (tok[None, None, :] < nvalid[:, g, :, None]))
        ok = ok.reshape(Bt, mx * P, 1)
        t = tau_f[:, g * G:(g + 1) * G].double()[:, None, :]
        x = (z.double() - t).clamp(min=0.0) ** gamma
        kept[:, g * G:(g + 1) * G] = torch.where(ok, x, torch.zeros_like(x)).sum(dim=1)
        del kt, z, x
    delta = (1.0 - kept).clamp(min=0.0)
    # a head's support is recovered when the kept pages hold all of its
    # full-cache entmax mass (to the resolution of the fp32 scores)
    recovered = (delta <= 1e-5) & (sup_s == sup_f)
    res["support_recovery_rate"] = float(recovered.float().mean())
    res["entmax_dropped_mass"] = {"mean": float(delta.mean()), "max": float(delta.max()),
                                  "note": "1 - kept entmax mass at the full-cache tau (fp64 "
                                          "sum of fp32 scores, resolution ~1e-6)"}
    return res


def time_steps(layers, steps, warmup, graph):
    import torch
    R = len(layers)
    for i in range(warmup):
        layers[i % R].step()
    torch.cuda.synchronize()
    if graph:
        graphs = []
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for L in layers:          # warm the capture stream
                L.step()
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        # one graph per pass over the R layers (as a decode loop would capture
        # its layers), plus one graph per layer for a remainder of K mod R
        full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(full):
            for L in layers:
                L.step()
        for L in layers[:steps % R]:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                L.step()
            graphs.append(g)
        for _ in range(max(1, warmup // R)):
            full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps // R):
            full.replay()
        for g in graphs:
            g.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(end) / steps, wall
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        layers[i % R].step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def step_distribution(layers, n, graph):
    """Median / p10 / p90 (ms) of n individually timed steps (HIP events around
    each step; with graph=True each step is the replay of that layer's captured
    step, so the figure includes one graph launch)."""
    import torch
    R = len(layers)
    graphs = []
    if graph:
        for L in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                L.step()
            graphs.append(g)
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    marks = []
    for i in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        if graph:
            graphs[i % R].replay()
        else:
            layers[i % R].step()
        b.record()
        marks.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in marks)
    pick = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    del graphs
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "steps": n}


def time_stages(layers, steps, graph, names=None):
    """Average duration (ms) of one launch of each entry point.

    With graphs: one graph per entry point holding its launches for every
    rotated layer in turn; it is replayed between two HIP events on the launch
    stream, so the figure is the kernel time plus the dispatch gap between two
    graph nodes.  Without graphs: events around every eager launch.
    """
    import torch
    names = layers[0].stages if names is None else names
    R = len(layers)
    res = {}
    if graph:
        reps = max(2, steps // R)
        for n in names:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for L in layers:
                    getattr(L, n)()
            g.replay()
            g.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            res[n] = a.elapsed_time(b) / (reps * R)
            del g
        return res
    acc = {n: 0.0 for n in names}
    evs = []
    for i in range(steps):
        L = layers[i % R]
        marks = []
        for n in names:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            getattr(L, n)()
            b.record()
            marks.append((n, a, b))
        evs.append(marks)
    torch.cuda.synchronize()
    for marks in evs:
        for n, a, b in marks:
            acc[n] += a.elapsed_time(b)
    return {n: acc[n] / steps for n in names}


def cpu_baseline(layer, budget_s):
    """The oracle as it stands, timed on host cores over a bounded sample of pairs."""
    from threadpoolctl import threadpool_limits
    from oracle import pipeline
    w = layer.w
    pairs = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    # spread the sample over the batch
    order = pairs[::max(1, len(pairs) // 16)] + pairs
    seen, sample = set(), []
    for p in order:
        if p not in seen:
            seen.add(p)
            sample.append(p)
    timed, done = 0.0, 0
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        for b, g in sample:
            t = {}
            pipeline.run_pair(layer.inp, b, g, w.policy, timings=t)
            timed += t.get("score", 0) + t.get("select", 0) + t.get("decode", 0)
            done += 1
            if time.perf_counter() - t_start > budget_s:
                break
    per_step = timed / done * len(pairs)
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (row, KV head) pairs of one {w.name} step "
                      f"(score + select + decode, metadata prebuilt), scaled linearly to "
                      f"all pairs; fp64 numpy, 1 BLAS thread",
            "seconds_per_step": per_step, "host": host_cpu()}


def host_cpu():
    """The host the CPU baseline ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = None
    return {"nproc": os.cpu_count(), "usable_cpus": avail, "cpu_model": model,
            "blas_threads": 1}


def workload_config(w, R, graph, inp):
    lens = inp["lens"]
    ctx = lens[0] if w.lens_range is None else f"U[{w.lens_range[0]},{w.lens_range[1]}]"
    return {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "context": ctx,
            "page_size": w.page_size, "kv_dtype": w.kv_dtype, "alpha": w.alpha,
            "policy": w.policy, "top_k": w.top_k if w.policy == "topk" else None,
            "delta": w.delta if w.policy in ("gauss", "gauss_est", "gauss_mass") else None,
            "q_std_x_sqrt_d": round(w.q_std * math.sqrt(w.head_dim), 6),
            "layers_rotated": R, "hip_graph": graph,
            "graph_scope": "one graph per pass over the rotated layers" if graph else None}


def run(w, args, dev, emit_cpu=True, light=False):
    """Time one workload's step.  light: a shorter run for the extra workloads
    reported with the headline line (fewer steps, no per-step distribution)."""
    import torch
    R = args.layers
    if R <= 0:
        probe = Layer(w, 0, dev)
        per_layer = stage_bytes_after_step(probe)["kv_bytes"]
        R = max(2, min(16, math.ceil((1 << 30) / max(per_layer, 1))))
        layers = [probe] + [Layer(w, 7919 * (i + 1), dev) for i in range(R - 1)]
    else:
        layers = [Layer(w, 7919 * i, dev) for i in range(R)]
    graph = not args.no_graph
    steps = min(args.steps, 100) if light else args.steps
    ms, wall = time_steps(layers, steps, min(args.warmup, 10) if light else args.warmup, graph)
    dist = None if light else {"graph": step_distribution(layers, 100, True),
                               "eager": step_distribution(layers, 100, False)}
    nst = max(20, min(steps, 400))
    stages = time_stages(layers, nst, graph)
    refresh_ms = time_stages(layers, nst, graph, ["refresh"])["refresh"]
    append_ms = time_stages(layers, nst, graph, ["append"])["append"]
    copy_gbps = measured_copy_gbps(dev)
    nb = stage_bytes(layers[0])
    eff = nb["kv_bytes"] / (ms * 1e-3) / 1e9
    dom = max(stages, key=lambda n: stages[n])
    dom_bytes = nb[dom]
    achieved = dom_bytes / (stages[dom] * 1e-3) / 1e9
    rec = {
        "metric": METRIC, "value": 1000.0 / ms, "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic", "config": workload_config(w, R, graph, layers[0].inp),
        "effective_kv_gbps": eff, "hbm_frac": eff / HBM_PEAK_GBPS,
        "measured_copy_gbps": copy_gbps, "frac_of_measured_copy": eff / copy_gbps,
        "kv_bytes_per_step": nb["kv_bytes"], "full_cache_bytes": nb["full_cache"],
        "read_fraction_of_full_cache": nb["kv_bytes"] / nb["full_cache"],
        "stage_ms": stages, "stage_bytes": {k: nb[k] for k in stages},
        "host_wall_ms_per_step": wall * 1000.0 / steps,
        "last_page_refresh": {"ms": refresh_ms, "bytes": nb["refresh"],
                              "gbps": nb["refresh"] / (refresh_ms * 1e-3) / 1e9,
                              "note": "build_page_meta of each row's last page, timed "
                                      "separately, not part of the step"},
        "append_token": {"ms": append_ms, "bytes": nb["append"],
                         "gbps": nb["append"] / (append_ms * 1e-3) / 1e9,
                         "note": "ekv_append_token of one token per row (K/V rows written, "
                                 "page metadata updated), timed separately"},
        "roofline": {"kernel": ENTRY_POINT[dom], "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(ENTRY_POINT[dom], w.name),
                     "algorithmic_bytes": dom_bytes, "launch_ms": stages[dom]},
    }
    if dist is not None:
        rec["step_ms_distribution"] = dict(dist, note="100 steps each timed by its own HIP "
                                           "events: graph = replay of the layer's captured "
                                           "step, eager = the step's launches")
    if light:
        rec["steps"] = steps
    rec["diagnostics"] = diagnostics(layers[0])
    if emit_cpu and args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(layers[0], args.cpu_seconds)
    del layers
    torch.cuda.empty_cache()
    return rec


def measured_copy_gbps(dev, mib=1024, reps=5):
    """HBM rate of a plain device-to-device copy on this GPU (bytes read + written per second)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    return 2 * n / sec / 1e9


def kernel_source_files(entry):
    """The HIP file of an entry point and every device-code header it includes (the
    library's own sources; the public C header, which declares the host interface
    and holds no device code, is left out)."""
    import re
    dirs = [os.path.join(HERE, "sparse_kv_cache_page_amd", "csrc")]
    todo, seen = [KERNEL_SOURCES[entry]], []
    while todo:
        name = todo.pop(0)
        if name in seen:
            continue
        path = next((os.path.join(d, name) for d in dirs if os.path.exists(os.path.join(d, name))), None)
        if path is None:
            continue  # a system header
        seen.append(name)
        with open(path) as fh:
            todo += re.findall(r'^#include "([^"]+)"', fh.read(), flags=re.M)
    return [(n, next(os.path.join(d, n) for d in dirs if os.path.exists(os.path.join(d, n))))
            for n in seen]


def kernel_source_hash(entry):
    """sha256 over the sources an entry point's kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for name, path in kernel_source_files(entry):
        with open(path, "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_traffic(entry, workload):
    """HBM bytes per launch from recorded FETCH_SIZE/WRITE_SIZE runs, or None.

    None when nothing is recorded for this entry point and workload, or when
    the kernel sources changed after the counters were taken.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    for r in rec.get("entries", []):
        if r.get("entry") == entry and r.get("workload") == workload:
            if r.get("source_sha256") != kernel_source_hash(entry):
                return None
            return r.get("hbm_bytes_per_launch")
    return None


def counter_summary(path):
    """Per-kernel mean of each counter in a rocprofv3 counter_collection.csv."""
    import csv
    import re
    agg = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = re.sub(r"\(anonymous namespace\)::", "", row["Kernel_Name"])
            name = re.sub(r"\(.*$", "", name.replace("void ", ""))[:100]
            key = (name, row["Counter_Name"])
            a = agg.setdefault(key, [0, 0.0, 0.0])
            a[0] += 1
            a[1] += float(row["Counter_Value"])
            a[2] += (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
    print(f"{'kernel':100s} {'counter':12s} {'dispatches':>10s} {'mean value':>14s} {'mean us':>9s}")
    for (name, ctr), (n, v, t) in sorted(agg.items(), key=lambda kv: -kv[1][2]):
        print(f"{name:100s} {ctr:12s} {n:10d} {v / n:14.1f} {t / n:9.2f}")


def stage_bytes_after_step(layer):
    import torch
    layer.step()
    torch.cuda.synchronize()
    return stage_bytes(layer)


def build_workload(args):
    from sparse_kv_cache_page_amd import workloads as wl
    w = wl.CONFIGS[args.config]
    kw = {}
    if args.alpha is not None:
        kw["alpha"] = args.alpha
    if args.policy is not None:
        kw["policy"] = args.policy
    if args.top_k is not None:
        kw["top_k"] = args.top_k
    if args.temperature is not None:
        kw["q_std"] = args.temperature / math.sqrt(w.head_dim)
    return wl.variant(w, **kw) if kw else w


def sweep(dev, steps=100, warmup=10):
    """batch x ctx sweep on the gqa decode heads (32 query / 8 KV heads, d 128, page 16,
    bf16, alpha 1.5), batch 1/8/32/64 x context 8k/32k/128k, top-k = 1/8 of the pages:
    one graph-replayed step per point, with its algorithmic bytes (the same
    accounting as the main line)."""
    import gc
    import torch
    from sparse_kv_cache_page_amd import workloads as wl
    out = []
    for B in (1, 8, 32, 64):
        for ctx in (8192, 32768, 131072):
            w = wl.variant("gqa", batch=B, seq_len=ctx, top_k=ctx // 16 // 8,
                           name=f"gqa_b{B}_ctx{ctx}")
            probe = Layer(w, 0, dev)
            per_layer = stage_bytes_after_step(probe)["kv_bytes"]
            R = max(2, min(16, math.ceil((1 << 30) / max(per_layer, 1))))
            layers = [probe] + [Layer(w, 7919 * (i + 1), dev) for i in range(R - 1)]
            ms, _ = time_steps(layers, steps, warmup, True)
            nb = stage_bytes(layers[0])
            eff = nb["kv_bytes"] / (ms * 1e-3) / 1e9
            out.append({"batch": B, "context": ctx, "top_k": w.top_k, "ms_per_step": ms,
                        "steps_per_s": 1000.0 / ms, "effective_kv_gbps": eff,
                        "hbm_frac": eff / HBM_PEAK_GBPS,
                        "read_fraction_of_full_cache": nb["kv_bytes"] / nb["full_cache"]})
            print(f"[sweep] B={B} ctx={ctx}: {1000.0 / ms:.1f} steps/s, {eff:.0f} GB/s",
                  file=sys.stderr, flush=True)
            del layers, probe
            gc.collect()
            torch.cuda.empty_cache()
    return out


def comparison(w, args, dev, step_ms, copy_gbps):
    """Softmax decode over the same selected pages and over the full cache, and the
    full-cache entmax decode, on the same layers (graph-replayed launches); the
    dropped softmax mass and the sparse-vs-full output error of both mappings on
    the first layer."""
    import gc
    import torch
    R = max(2, args.layers) if args.layers > 0 else 4
    layers = [Layer(w, 7919 * i, dev) for i in range(R)]
    for L in layers:
        L.step()
        L._cmp_buffers()
    names = ["softmax_sel", "softmax_full", "entmax_full"]
    t = time_stages(layers, 40, not args.no_graph, names)
    L0 = layers[0]
    L0.step()
    for n in names:
        getattr(L0, n)()
    torch.cuda.synchronize()
    c = L0.cmp
    # the dropped softmax mass directly: softmax over the pages NOT selected,
    # delta = exp(lse_dropped - lse_full) (1 - exp(lse_sel - lse_full) loses
    # everything below fp32 resolution of lse)
    from sparse_kv_cache_page_amd import binding as Bd
    s0, dec0, inp0 = L0.shape, L0.dec, L0.inp
    mp = s0.max_pages_per_seq
    npg = torch.tensor(inp0["npages"], device=dec0.sel.device)
    idx = torch.arange(mp, device=dec0.sel.device)
    # selected pages marked in a table with one spare column for the unused slots
    taken = torch.zeros(s0.batch, s0.num_kv_heads, mp + 1, dtype=torch.bool, device=idx.device)
    live = idx[None, None, :] < dec0.n_sel.long()[:, :, None]
    taken.scatter_(2, torch.where(live, dec0.sel.long().clamp(0, mp - 1),
                                  torch.full_like(dec0.sel.long(), mp)), True)
    dropped = (~taken[:, :, :mp]) & (idx[None, None, :] < npg[:, None, None])
    # dropped pages first, ascending (stable sort on "not dropped")
    comp = torch.sort((~dropped).to(torch.int8), dim=2, stable=True).indices.to(torch.int32)
    n_comp = dropped.sum(dim=2).to(torch.int32)
    lse_d = torch.empty_like(c["lse_full"])
    o_d = torch.empty_like(c["o_sm_full"])
    ws_d = torch.empty(Bd.softmax_workspace_bytes(s0, 0), dtype=torch.uint8, device=idx.device)
    Bd.softmax_decode(s0, inp0["q"], L0.w.scale, inp0["K"], inp0["V"], inp0["block_table"],
                      inp0["seq_lens"], o_d, ws_d, sel=comp.contiguous(), n_sel=n_comp,
                      max_sel=mp, lse=lse_d)
    torch.cuda.synchronize()
    delta = torch.exp(lse_d.double() - c["lse_full"].double()).flatten()

    def rel(a, b):
        return ((a - b).norm(dim=-1) / b.norm(dim=-1).clamp_min(1e-30)).flatten()

    e_ent = rel(L0.dec.out, c["o_ent_full"])
    e_sm = rel(c["o_sm_sel"], c["o_sm_full"])
    nb = stage_bytes(L0)
    full_kv = nb["full_cache"]
    res = {
        "ms": t,
        "entmax_step_ms": step_ms,
        "speedup_vs_softmax_full_cache": t["softmax_full"] / step_ms,
        "speedup_vs_entmax_full_cache": t["entmax_full"] / step_ms,
        "softmax_full_cache_gbps": full_kv / (t["softmax_full"] * 1e-3) / 1e9,
        # against a softmax decode that streamed the full cache at the measured
        # device-copy rate (an upper bound for any full-cache decode here)
        "speedup_vs_full_cache_read_at_copy_rate":
            full_kv / (copy_gbps * 1e9) / (step_ms * 1e-3),
        "softmax_full_cache_hbm_frac": full_kv / (t["softmax_full"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "softmax_dropped_mass": {"mean": float(delta.mean()), "max": float(delta.max()),
                                 "min": float(delta.min()),
                                 "note": "exp(lse of the dropped pages - lse of all pages)"},
        "sparse_vs_full_output_rel_err": {
            "entmax": {"median": float(e_ent.median()), "max": float(e_ent.max())},
            "softmax": {"median": float(e_sm.median()), "max": float(e_sm.max())}},
        "note": "same layers and selected pages; full-cache bytes = every valid K and V row",
    }
    print(f"[comparison] step {step_ms * 1000:.1f} us; softmax same pages "
          f"{t['softmax_sel'] * 1000:.1f} us, softmax full {t['softmax_full'] * 1000:.1f} us, "
          f"entmax full {t['entmax_full'] * 1000:.1f} us", file=sys.stderr, flush=True)
    del layers
    gc.collect()
    torch.cuda.empty_cache()
    return res


def extra_workloads(args, dev):
    """The larger single-GPU workloads, reported with the headline line: ragged
    (batch 64, lengths U[4096, 65536], top-512), stress (batch 32, context
    131072, 64/8 heads, page 32, alpha 1.25) with top-512 pages and with the
    full-cache dense pass, and one 1M-token row (4/1 heads, top-8192 pages and
    the dense pass).  Each: steps/s, effective KV bandwidth, per entry
    point times and bytes, the roofline of its dominant entry point and the
    step diagnostics."""
    import gc
    import torch
    from sparse_kv_cache_page_amd import workloads as wl
    out = []
    for w in (wl.CONFIGS["ragged"], wl.CONFIGS["stress"],
              wl.variant("stress", policy="dense", name="stress_dense"),
              wl.CONFIGS["long1m"], wl.variant("long1m", policy="dense", name="long1m_dense")):
        print(f"[workloads] {w.name}", file=sys.stderr, flush=True)
        r = run(w, args, dev, emit_cpu=False, light=True)
        keep = ("config", "value", "unit", "ms_per_step", "steps", "effective_kv_gbps",
                "hbm_frac", "frac_of_measured_copy", "kv_bytes_per_step", "full_cache_bytes",
                "read_fraction_of_full_cache", "stage_ms", "stage_bytes", "roofline",
                "diagnostics")
        out.append({k: r[k] for k in keep if k in r})
        gc.collect()
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (every "
              "(row, KV head) pair is independent, so rows or KV heads would be split across "
              "GPUs with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}))
        return
    from sparse_kv_cache_page_amd import binding
    binding.load_library()
    dev = torch.device("cuda:0")
    w = build_workload(args)
    rec = run(w, args, dev)
    if (w.name == "gqa" or (args.comparison and w.policy == "topk")) and not args.no_comparison:
        rec["comparison"] = comparison(w, args, dev, rec["ms_per_step"],
                                       rec["measured_copy_gbps"])
    if w.name == "gqa" and not args.no_extra:
        rec["workloads"] = extra_workloads(args, dev)
    if w.name == "gqa" and not args.no_sweep:
        rec["sweep"] = sweep(dev)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
