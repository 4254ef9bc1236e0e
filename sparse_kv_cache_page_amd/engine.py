"""Buffers and call sequence of one paged entmax decode step.

`PagedEntmaxDecoder` owns the device buffers a decode step needs for one cache
shape (page metadata, page bounds, selections, decode workspace; all torch
allocations, made once) and issues the library calls in order:

    build_page_meta   (once per prefill; span=1 refresh of the last page per step)
    score_pages -> select_pages -> entmax_decode   (every decode step)

This is the pipeline of the EntmaxKV summary page, §2 "Méthodologie": score
pages from lightweight per-page metadata, select candidates, then run sparse
alpha-entmax over the selected pages only.  All arithmetic happens in the HIP
library; this class only allocates and sequences.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B
from .binding import CacheShape


class PagedEntmaxDecoder:
    def __init__(self, shape: CacheShape, *, policy: str = "topk", top_k: int = 256,
                 alpha: float = 1.5, scale: float = 1.0, delta: float = 0.1,
                 device: Optional[torch.device] = None, fused: bool = False,
                 prune: Optional[bool] = None):
        if policy not in ("topk", "gauss", "gauss_est", "gauss_mass", "dense"):
            raise ValueError("policy must be 'topk', 'gauss', 'gauss_est', 'gauss_mass' or "
                             "'dense'")
        self.shape = s = shape
        self.policy = policy
        self.top_k = int(top_k)
        self.alpha = float(alpha)
        self.scale = float(scale)
        self.delta = float(delta)
        dev = torch.device(device) if device is not None else torch.device("cuda")
        self.device = dev
        Bt, Hq, Hkv, d, mp, Np = (s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                  s.max_pages_per_seq, s.num_phys_pages)
        gauss = policy in ("gauss", "gauss_est", "gauss_mass")
        self.kmin = torch.empty(Np, Hkv, d, dtype=s.kv_dtype, device=dev)
        self.kmax = torch.empty(Np, Hkv, d, dtype=s.kv_dtype, device=dev)
        md = s.moments_dtype
        self.mean = torch.empty(Np, Hkv, d, dtype=md, device=dev) if gauss else None
        self.var = torch.empty(Np, Hkv, d, dtype=md, device=dev) if gauss else None
        self.ubg = torch.empty(Bt, Hkv, mp, dtype=torch.float32, device=dev)
        # per-head page bounds: read by the box-bound Gaussian rule, and by the
        # decode's page pruning.  Pruning is on by default for top-k only: the
        # Gaussian rules keep a page only if its estimated maximum reaches
        # tau_hat - delta, and tau_hat tracks tau >= z_max - 1, so the pages
        # they keep already lie near z_max - 1 and the probe launch would find
        # nothing to skip (prune=True still forces it)
        if prune is None:
            prune = policy == "topk"
        self.prune = bool(prune) and policy != "dense"
        self.ub = (torch.empty(Bt, Hkv, mp, Hq // Hkv, dtype=torch.float32, device=dev)
                   if policy == "gauss" or self.prune else None)
        self.zlb = torch.empty(Bt, Hq, dtype=torch.float32, device=dev) if self.prune else None
        self.gm = torch.empty(Bt, Hq, mp, dtype=torch.float64, device=dev) if gauss else None
        self.gv = torch.empty(Bt, Hq, mp, dtype=torch.float64, device=dev) if gauss else None
        self.tau_hat = torch.empty(Bt, Hq, dtype=torch.float64, device=dev) if gauss else None
        self.sel = torch.empty(Bt, Hkv, mp, dtype=torch.int32, device=dev)
        self.n_sel = torch.empty(Bt, Hkv, dtype=torch.int32, device=dev)
        self.out = torch.empty(Bt, Hq, d, dtype=torch.float32, device=dev)
        self.tau = torch.empty(Bt, Hq, dtype=torch.float32, device=dev)
        self.n_support = torch.empty(Bt, Hq, dtype=torch.int32, device=dev)
        # the box scorer's best-page hints (top-k with pruning): ekv_score_box_pages
        # writes them, ekv_topk_decode reads them
        self.hint = (torch.empty(max(B.score_hint_bytes(s), 256), dtype=torch.uint8, device=dev)
                     if policy == "topk" and self.prune else None)
        self.max_sel = min(self.top_k, mp) if policy == "topk" else mp
        ws_bytes = B.decode_workspace_bytes(s, self.max_sel)
        if policy == "topk":
            # the same workspace serves ekv_topk_decode (a little larger)
            ws_bytes = max(ws_bytes, B.topk_decode_workspace_bytes(s, self.top_k))
        self.ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        # the fused step (top-k only) keeps arrival counters in its workspace:
        # zero-filled once here, left zeroed by every call
        self.fused = bool(fused) and policy == "topk"
        if self.fused:
            self.step_ws = torch.zeros(B.step_workspace_bytes(s, self.top_k), dtype=torch.uint8,
                                       device=dev)
            self.sel_ws = torch.zeros(B.score_select_workspace_bytes(s), dtype=torch.uint8,
                                      device=dev)

    # -- metadata -----------------------------------------------------------
    def build_meta(self, K, block_table, seq_lens, first_page=None, span: int = 0):
        B.build_page_meta(self.shape, K, block_table, seq_lens, self.kmin, self.kmax,
                          self.mean, self.var, first_page=first_page, span=span)

    def append(self, k_new, v_new, K, V, block_table, seq_lens):
        """Write each row's new token (at seq_lens - 1, already counted) into the
        cache and update its page's metadata, in one launch."""
        B.append_token(self.shape, k_new, v_new, block_table, seq_lens, K, V, self.kmin,
                       self.kmax, self.mean, self.var)

    # -- one decode step ----------------------------------------------------
    def score(self, q, block_table, seq_lens):
        B.score_pages(self.shape, q, self.scale, self.kmin, self.kmax, block_table, seq_lens,
                      self.ubg, ub=self.ub, mean=self.mean, var=self.var, gm=self.gm, gv=self.gv)

    def select(self, seq_lens):
        if self.policy == "topk":
            B.select_pages(self.shape, seq_lens, B.EKV_SELECT_TOPK, self.top_k, self.alpha,
                           self.delta, self.ubg, self.sel, self.n_sel)
        elif self.policy in ("gauss", "gauss_est", "gauss_mass"):
            pol = {"gauss": B.EKV_SELECT_GAUSS, "gauss_est": B.EKV_SELECT_GAUSS_EST,
                   "gauss_mass": B.EKV_SELECT_GAUSS_MASS}[self.policy]
            B.select_pages(self.shape, seq_lens, pol, self.top_k, self.alpha, self.delta,
                           self.ubg, self.sel, self.n_sel, ub=self.ub, gm=self.gm, gv=self.gv,
                           tau_hat=self.tau_hat)

    def decode(self, q, K, V, block_table, seq_lens):
        dense = self.policy == "dense"
        B.entmax_decode(self.shape, q, self.scale, self.alpha, K, V, block_table, seq_lens,
                        self.out, self.ws, sel=None if dense else self.sel,
                        n_sel=None if dense else self.n_sel, max_sel=self.max_sel, tau=self.tau,
                        n_support=self.n_support, ub=self.ub if self.prune else None,
                        zlb=self.zlb)

    def score_box(self, q, block_table, seq_lens, K=None, refresh_last_page: bool = False):
        """Box bounds (and the best-page hints) of the top-k step, one launch."""
        B.score_box_pages(self.shape, q, self.scale, block_table, seq_lens, self.kmin, self.kmax,
                          self.ubg, ub=self.ub, hint=self.hint, K=K,
                          refresh_last_page=refresh_last_page)

    def topk_decode(self, q, K, V, block_table, seq_lens, use_hint: bool = False):
        """Top-k selection from the group bounds and the (pruned) decode over it, in
        one entry point (after score(), or after score_box() with use_hint)."""
        B.topk_decode(self.shape, q, self.scale, self.alpha, K, V, block_table, seq_lens,
                      self.top_k, self.ubg, self.sel, self.n_sel, self.out, self.ws,
                      ub=self.ub if self.prune else None, tau=self.tau,
                      n_support=self.n_support,
                      hint=self.hint if (use_hint and self.prune) else None)

    def score_select(self, q, K, block_table, seq_lens, refresh_last_page: bool = False):
        """[last-page refresh] + scores + top-k in one fused launch."""
        B.score_select_pages(self.shape, q, self.scale, K, block_table, seq_lens, self.top_k,
                             self.kmin, self.kmax, self.ubg, self.sel, self.n_sel, self.sel_ws,
                             refresh_last_page=refresh_last_page, ub=self.ub)

    def fused_step(self, q, K, V, block_table, seq_lens, refresh_last_page: bool = False):
        """[last-page refresh] + score + top-k + decode in two fused launches."""
        B.decode_step(self.shape, q, self.scale, self.alpha, K, V, block_table, seq_lens,
                      self.top_k, self.kmin, self.kmax, self.ubg, self.sel, self.n_sel, self.out,
                      self.step_ws, refresh_last_page=refresh_last_page, tau=self.tau,
                      n_support=self.n_support)
        return self.out, self.tau

    def step(self, q, K, V, block_table, seq_lens):
        """score -> select -> decode; returns (out, tau) views of the owned buffers."""
        if self.fused:
            return self.fused_step(q, K, V, block_table, seq_lens)
        if self.policy != "dense":
            self.score(q, block_table, seq_lens)
            self.select(seq_lens)
        self.decode(q, K, V, block_table, seq_lens)
        return self.out, self.tau
