"""Seeded sweep over random small configurations (GPU vs oracle on every pair).

Each case draws the batch, group size, head dim, K/V dtype, page size, row
lengths (empty rows included), alpha, policy and its parameter, and the
metadata format, runs the whole step on the GPU, and checks every (row, KV
head) pair against the oracle with the usual tolerances (selections exact).
"""
import numpy as np
import pytest

from sparse_kv_cache_page_amd import workloads as wl

from gpu_util import check_pair, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def draw(seed):
    r = np.random.default_rng(900 + seed)
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 3]))
    d = int(r.choice([64, 128]))
    P = int(r.choice([1, 2, 4, 8, 16, 32, 64]))
    policy = str(r.choice(["topk", "topk", "dense", "gauss", "gauss_est", "gauss_mass"]))
    gauss = policy.startswith("gauss")
    alpha = float(r.choice([2.0, 1.5, 4.0 / 3.0, 1.25])) if gauss else \
        float(r.choice([1.1, 1.25, 1.5, 2.0, 3.0]))
    batch = int(r.integers(1, 5))
    lens = [int(r.integers(1, 1500)) for _ in range(batch)]
    if batch > 1 and r.random() < 0.3:
        lens[int(r.integers(0, batch))] = 0          # an idle slot
    kv = "f32" if r.random() < 0.25 else "bf16"
    w = wl.Workload(name="rand", batch=batch, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                    head_dim=d, page_size=P, seq_len=max(lens), kv_dtype=kv,
                    q_std=float(r.uniform(0.5, 3.0)) / np.sqrt(d), scale=1.0, alpha=alpha,
                    policy=policy, top_k=int(r.integers(1, 200)),
                    delta=float(r.choice([1e-4, 1e-3, 1e-2])) if policy == "gauss_mass"
                    else float(r.choice([0.0, 0.1, 0.5])),
                    planted_per_kv_head=0 if gauss else int(r.choice([0, 4, 16])),
                    clusters=int(r.choice([8, 32])) if gauss else 0,
                    moments_bf16=bool(gauss and r.random() < 0.3),
                    permute_pool=bool(r.random() < 0.5), seed=int(r.integers(1, 1 << 30)))
    return w, lens


@pytest.mark.parametrize("seed", range(64))
def test_random_configuration(seed):
    w, lens = draw(seed)
    print(f"[random {seed}] {w}", flush=True)
    inp = wl.make_inputs(w, device=DEV, lens=lens)
    gpu = run_gpu(inp, w.policy)
    for b in range(w.batch):
        if lens[b] == 0:
            continue
        for g in range(w.num_kv_heads):
            check_pair(inp, gpu, b, g, w.policy)
    if w.policy == "topk":
        # the fused step (scores + top-k in one launch, then the pruned
        # decode) equals the separate calls bit for bit
        import torch
        from sparse_kv_cache_page_amd.engine import PagedEntmaxDecoder
        from gpu_util import cache_shape
        f = PagedEntmaxDecoder(cache_shape(inp), policy="topk", top_k=w.top_k, alpha=w.alpha,
                               scale=w.scale, fused=True)
        f.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
        f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
        torch.cuda.synchronize()
        assert torch.equal(f.n_sel, gpu["n_sel"])
        for k in ("out", "tau", "n_support"):
            assert torch.equal(torch.nan_to_num(f.__dict__[k], nan=-9.0),
                               torch.nan_to_num(gpu[k], nan=-9.0)), k
