"""Seeded synthetic decode workloads for the paged entmax decode path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no scores, bounds, thresholds or selections).  Both the
HIP path (tests, bench) and the CPU oracle (tests) consume what it produces, so
the oracle always sees exactly the bits the GPU sees.

The shapes follow the long-context decode workloads of the EntmaxKV summary
page (gist.science, paper 2605.21649), §4 "Résultats Clés": passkey-like
needles planted at any depth, contexts up to 131072 tokens, ragged batches.
The datasets themselves (RULER, passkey, PG19) are not used; these synthetic
draws stand in for them.

Layout produced (all torch tensors on the requested device):
  q            fp32  [B][Hq][d]
  K, V         bf16 or fp32  [Np][Hkv][P][d]   (one contiguous P x d tile per
                                                 physical page and KV head)
  block_table  int32 [B][maxP]   logical page -> physical page (-1 = unused)
  seq_lens     int32 [B]
Padding slots (token positions >= L_b inside a sequence's last page) hold
sentinel values so that a kernel that reads them as keys or values produces
visibly wrong results.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

# Value written into K padding slots (finite, representable in bf16) and into
# V padding slots.  A correct implementation never reads either.
K_PAD_SENTINEL = 8192.0
V_PAD_SENTINEL = float("nan")


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    seq_len: int = 0                 # fixed length for every row (if lens_range is None)
    lens_range: Optional[tuple] = None  # (lo, hi) inclusive uniform lengths
    kv_dtype: str = "bf16"           # "bf16" or "f32"
    q_std: float = 1.0               # per-coordinate std of q
    scale: float = 1.0               # score scale passed to the library
    alpha: float = 1.5
    policy: str = "topk"             # "topk" | "gauss" | "gauss_est" | "gauss_mass" | "dense"
    top_k: int = 256
    delta: float = 0.1
    planted_per_kv_head: int = 0     # planted high-score keys per (row, KV head)
    planted_literal: bool = False    # True: k = 3 q + noise; False: k = 3 q / q_std + noise
    planted_noise: float = 0.1
    moments_bf16: bool = False       # page mean/variance stored as bf16 (else fp32)
    clusters: int = 0                # >0: clustered keys (centroids per KV head)
    cluster_sigma: float = 0.5
    permute_pool: bool = False
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _cfg(**kw) -> Workload:
    return Workload(**kw)


# The five workload shapes.  Readings of under-specified points:
#  * scale: 1/sqrt(d) for the tiny case (raw N(0,1) query), 1 elsewhere (the
#    query already carries the temperature 2/sqrt(d)).
#  * planted keys: 3 q_h / q_std + N(0, 0.1^2), round-robin over the group's
#    query heads, at distinct uniform positions in [0, L_b).
#  * clustered keys: 64 centroids ~ N(0, I) per KV head, one per page, sigma 0.5.
CONFIGS = {
    "tiny": _cfg(name="tiny", batch=1, num_q_heads=1, num_kv_heads=1, head_dim=64,
                 page_size=16, seq_len=4096, kv_dtype="f32", q_std=1.0,
                 scale=0.125, alpha=1.5, policy="topk", top_k=32,
                 planted_per_kv_head=8, seed=1001),
    "gqa": _cfg(name="gqa", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                page_size=16, seq_len=32768, kv_dtype="bf16", q_std=2.0 / math.sqrt(128),
                scale=1.0, alpha=1.5, policy="topk", top_k=256,
                planted_per_kv_head=64, seed=2002),
    "gauss": _cfg(name="gauss", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  page_size=16, seq_len=32768, kv_dtype="bf16",
                  q_std=2.0 / math.sqrt(128), scale=1.0, alpha=2.0, policy="gauss",
                  delta=0.1, clusters=64, cluster_sigma=0.5, seed=3003),
    # gauss shapes, the expected-maximum estimate of a page's maximum score
    "gauss_est": _cfg(name="gauss_est", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      page_size=16, seq_len=32768, kv_dtype="bf16",
                      q_std=2.0 / math.sqrt(128), scale=1.0, alpha=2.0, policy="gauss_est",
                      delta=0.1, clusters=64, cluster_sigma=0.5, seed=3003),
    # gauss shapes, the expected-mass rule (delta is the mass threshold)
    "gauss_mass": _cfg(name="gauss_mass", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                       page_size=16, seq_len=32768, kv_dtype="bf16",
                       q_std=2.0 / math.sqrt(128), scale=1.0, alpha=2.0, policy="gauss_mass",
                       delta=1e-4, clusters=64, cluster_sigma=0.5, seed=3003),
    # the same with the compact metadata format (bf16 page mean / variance)
    "gauss_mass_m16": _cfg(name="gauss_mass_m16", batch=8, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, page_size=16, seq_len=32768, kv_dtype="bf16",
                           q_std=2.0 / math.sqrt(128), scale=1.0, alpha=2.0,
                           policy="gauss_mass", delta=1e-4, clusters=64, cluster_sigma=0.5,
                           moments_bf16=True, seed=3003),
    "ragged": _cfg(name="ragged", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                   page_size=16, lens_range=(4096, 65536), kv_dtype="bf16",
                   q_std=2.0 / math.sqrt(128), scale=1.0, alpha=1.5, policy="topk",
                   top_k=512, planted_per_kv_head=64, permute_pool=True, seed=4004),
    # one 1M-token row (the long-context point of the EntmaxKV page, §4): one
    # KV head with a group of four
    "long1m": _cfg(name="long1m", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                   page_size=16, seq_len=1 << 20, kv_dtype="bf16",
                   q_std=2.0 / math.sqrt(128), scale=1.0, alpha=1.5, policy="topk",
                   top_k=8192, planted_per_kv_head=64, seed=6006),
    "stress": _cfg(name="stress", batch=32, num_q_heads=64, num_kv_heads=8, head_dim=128,
                   page_size=32, seq_len=131072, kv_dtype="bf16",
                   q_std=3.99 / math.sqrt(128), scale=1.0, alpha=1.25, policy="topk",
                   top_k=512, seed=5005),
}

# Query temperature T (q = N(0,1) * T / sqrt(d)) that gives the stress shape a
# support of about 16 / 256 / 4096 tokens per head, per alpha.
STRESS_TEMPERATURE = {
    1.25: (3.99, 1.69, 0.662),
    1.5: (1.5, 0.313, 0.0596),
    2.0: (0.258, 0.0134, 0.000627),
}


def variant(base: str | Workload, **kw) -> Workload:
    w = CONFIGS[base] if isinstance(base, str) else base
    return dataclasses.replace(w, **kw)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_lengths(w: Workload) -> List[int]:
    if w.lens_range is None:
        return [w.seq_len] * w.batch
    g = _gen("cpu", w.seed + 1)
    lo, hi = w.lens_range
    return torch.randint(lo, hi + 1, (w.batch,), generator=g).tolist()


def make_inputs(w: Workload, device="cpu", lens: Optional[List[int]] = None) -> dict:
    """Draw one decode batch for workload `w` on `device`.

    Returns a dict with q, K, V, block_table, seq_lens and the host-side shape
    facts (num_phys_pages, max_pages, lens).  Identical seeds give identical
    tensors on the same device type.
    """
    B, Hq, Hkv, d, P = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    assert Hq % Hkv == 0
    G = Hq // Hkv
    lens = list(lens) if lens is not None else draw_lengths(w)
    # a row may be empty (an idle batch slot); at least one row holds tokens
    assert len(lens) == B and all(L >= 0 for L in lens) and max(lens) >= 1
    npages = [(L + P - 1) // P for L in lens]
    maxP = max(npages)
    Np = sum(npages)

    gcpu = _gen("cpu", w.seed + 2)
    # physical pool order
    if w.permute_pool:
        pool = torch.randperm(Np, generator=gcpu)
    else:
        pool = torch.arange(Np)
    block_table = torch.full((B, maxP), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        block_table[b, : npages[b]] = pool[off: off + npages[b]].to(torch.int32)
        off += npages[b]

    g = _gen(device, w.seed)
    kv_t = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32

    q = (torch.randn(B, Hq, d, generator=g, device=device, dtype=torch.float32) * w.q_std)

    def randn_pages(std=1.0):
        out = torch.empty(Np, Hkv, P, d, dtype=kv_t, device=device)
        step = max(1, (1 << 24) // (Hkv * P * d))
        for s in range(0, Np, step):
            e = min(Np, s + step)
            out[s:e] = (torch.randn(e - s, Hkv, P, d, generator=g, device=device) * std).to(kv_t)
        return out

    if w.clusters > 0:
        K = torch.empty(Np, Hkv, P, d, dtype=kv_t, device=device)
        cent = torch.randn(Hkv, w.clusters, d, generator=g, device=device)
        pick = torch.randint(0, w.clusters, (Np, Hkv), generator=g, device=device)
        step = max(1, (1 << 24) // (Hkv * P * d))
        hidx = torch.arange(Hkv, device=device)
        for s in range(0, Np, step):
            e = min(Np, s + step)
            c = cent[hidx[None, :], pick[s:e]]                       # [n][Hkv][d]
            noise = torch.randn(e - s, Hkv, P, d, generator=g, device=device)
            K[s:e] = (c[:, :, None, :] + w.cluster_sigma * noise).to(kv_t)
    else:
        K = randn_pages()
    V = randn_pages()

    if w.planted_per_kv_head > 0:
        n_pl = w.planted_per_kv_head
        bt_dev = block_table.to(device)
        for b in range(B):
            L = lens[b]
            m = min(n_pl, L)
            if m == 0:
                continue
            # distinct uniform positions per KV head
            pos = torch.stack([torch.randperm(L, generator=gcpu)[:m] for _ in range(Hkv)])  # [Hkv][m]
            heads = (torch.arange(Hkv)[:, None] * G + (torch.arange(m)[None, :] % G))  # [Hkv][m]
            qh = q[b, heads.reshape(-1).to(device)].reshape(Hkv, m, d)
            base = qh * 3.0 if w.planted_literal else qh * (3.0 / w.q_std)
            keys = base + w.planted_noise * torch.randn(Hkv, m, d, generator=g, device=device)
            pos_d = pos.to(device)
            phys = bt_dev[b, (pos_d // P).long()].long()               # [Hkv][m]
            gidx = torch.arange(Hkv, device=device)[:, None].expand(Hkv, m)
            K[phys, gidx, (pos_d % P).long()] = keys.to(kv_t)

    # sentinels in padding slots of each last page
    for b in range(B):
        L = lens[b]
        t0 = L - (npages[b] - 1) * P
        if t0 < P:
            pl = int(block_table[b, npages[b] - 1])
            K[pl, :, t0:, :] = K_PAD_SENTINEL
            V[pl, :, t0:, :] = V_PAD_SENTINEL

    return dict(
        q=q, K=K, V=V,
        block_table=block_table.to(device),
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        lens=lens, npages=npages, max_pages=maxP, num_phys_pages=Np,
        workload=w,
    )


def fresh_query(w: Workload, inputs: dict, seed: int) -> torch.Tensor:
    """A new query batch of the same distribution (used to vary selections across steps)."""
    dev = inputs["q"].device
    g = _gen(dev, seed)
    return torch.randn(w.batch, w.num_q_heads, w.head_dim, generator=g, device=dev,
                       dtype=torch.float32) * w.q_std

