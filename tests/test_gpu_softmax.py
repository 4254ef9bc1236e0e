"""GPU parity of the softmax comparison path (ekv_softmax_decode) against the
oracle's softmax decode, over the selected pages and over the full cache.

Tolerances: out relative L2 <= 1e-3 per query head (fp32 accumulation of
exactly widened keys and values, as for the entmax output); lse within
1e-5 (1 + |lse|) (fp32 scores of magnitude up to ~70 on planted keys);
the dropped mass 1 - exp(lse_sel - lse_full) within 2e-4 absolute.
"""
import numpy as np
import pytest
import torch

from oracle import pipeline
from sparse_kv_cache_page_amd import binding as B
from sparse_kv_cache_page_amd import workloads as wl

from gpu_util import cache_shape, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUT_TOL = 1e-3
LSE_RTOL = 1e-5
DELTA_TOL = 2e-4


def small(seed, **kw):
    base = dict(name="small", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                page_size=16, lens_range=(37, 1500), kv_dtype="bf16",
                q_std=2.0 / np.sqrt(128), scale=1.0, alpha=1.5, policy="topk", top_k=9,
                planted_per_kv_head=8, permute_pool=True, seed=seed)
    base.update(kw)
    return wl.Workload(**base)


def run_softmax(inp, sel=None, n_sel=None, max_sel=0):
    s = cache_shape(inp)
    w = inp["workload"]
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), device=DEV)
    lse = torch.full((s.batch, s.num_q_heads), float("nan"), device=DEV)
    ws = torch.empty(B.softmax_workspace_bytes(s, max_sel if sel is not None else 0),
                     dtype=torch.uint8, device=DEV)
    B.softmax_decode(s, inp["q"], w.scale, inp["K"], inp["V"], inp["block_table"],
                     inp["seq_lens"], out, ws, sel=sel, n_sel=n_sel, max_sel=max_sel, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


def check_softmax(inp, o_sel, lse_sel, o_full, lse_full, sel, n_sel, b, g):
    w = inp["workload"]
    G = w.group
    pages = None
    if sel is not None:
        pages = [int(x) for x in sel[b, g, : int(n_sel[b, g])].cpu().tolist()]
    ref = pipeline.softmax_pair(inp, b, g, pages)
    hs = slice(g * G, (g + 1) * G)
    for i, h in enumerate(range(g * G, (g + 1) * G)):
        assert rel_l2(o_sel[b, h], ref["o"][i]) <= OUT_TOL, (b, h)
        assert rel_l2(o_full[b, h], ref["o_full"][i]) <= OUT_TOL, (b, h)
        assert abs(lse_sel[b, h] - ref["lse"][i]) <= LSE_RTOL * (1 + abs(ref["lse"][i])), (b, h)
        assert abs(lse_full[b, h] - ref["lse_full"][i]) <= \
            LSE_RTOL * (1 + abs(ref["lse_full"][i])), (b, h)
    delta = 1.0 - np.exp(lse_sel[b, hs] - lse_full[b, hs])
    np.testing.assert_allclose(delta, ref["dropped_mass"], rtol=0, atol=DELTA_TOL)
    return ref


def topk_sel(inp):
    gpu = run_gpu(inp, "topk")
    return gpu["sel"], gpu["n_sel"]


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (16, 2)])
def test_softmax_shapes(kv_dtype, head_dim, heads):
    Hq, Hkv = heads
    w = small(71 + head_dim + Hq, kv_dtype=kv_dtype, head_dim=head_dim, num_q_heads=Hq,
              num_kv_heads=Hkv, q_std=2.0 / np.sqrt(head_dim))
    inp = wl.make_inputs(w, device=DEV)
    sel, n_sel = topk_sel(inp)
    o_s, l_s = run_softmax(inp, sel, n_sel, max_sel=w.top_k)
    o_f, l_f = run_softmax(inp)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            check_softmax(inp, o_s, l_s, o_f, l_f, sel, n_sel, b, g)


@pytest.mark.parametrize("page_size", [1, 2, 8, 32, 64])
def test_softmax_page_sizes(page_size):
    w = small(91 + page_size, page_size=page_size, lens_range=(5, 900),
              top_k=max(1, 150 // page_size))
    inp = wl.make_inputs(w, device=DEV)
    sel, n_sel = topk_sel(inp)
    o_s, l_s = run_softmax(inp, sel, n_sel, max_sel=w.top_k)
    o_f, l_f = run_softmax(inp)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            check_softmax(inp, o_s, l_s, o_f, l_f, sel, n_sel, b, g)


def test_softmax_long_rows_many_splits():
    # rows of ~20k tokens: the full-cache call runs tens of splits per pair,
    # the last one ragged.  No planted keys: with them the dropped softmax
    # mass is ~exp(-66), below what 1 - exp(lse_sel - lse_full) resolves in fp64
    w = small(101, batch=2, lens_range=None, top_k=200, planted_per_kv_head=0)
    inp = wl.make_inputs(w, device=DEV, lens=[19993, 7001])
    sel, n_sel = topk_sel(inp)
    o_s, l_s = run_softmax(inp, sel, n_sel, max_sel=w.top_k)
    o_f, l_f = run_softmax(inp)
    B_ = None
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            ref = check_softmax(inp, o_s, l_s, o_f, l_f, sel, n_sel, b, g)
            # §3: dropping any token drops softmax mass, and the output moves by
            # at most 2 B delta
            assert np.all(ref["dropped_mass"] > 0)
            B_ = ref["value_norm_bound"]
            G = w.group
            for i, h in enumerate(range(g * G, (g + 1) * G)):
                err = np.linalg.norm(o_s[b, h] - o_f[b, h])
                assert err <= 2 * B_ * ref["dropped_mass"][i] + 1e-3 * np.linalg.norm(o_f[b, h])


def test_softmax_empty_rows_and_bound():
    w = small(111, batch=5, lens_range=None)
    inp = wl.make_inputs(w, device=DEV, lens=[0, 700, 0, 33, 1500])
    sel, n_sel = topk_sel(inp)
    o_s, l_s = run_softmax(inp, sel, n_sel, max_sel=w.top_k)
    o_f, l_f = run_softmax(inp)
    for b in (0, 2):
        assert np.all(o_s[b] == 0) and np.all(o_f[b] == 0)
        assert np.all(np.isneginf(l_s[b])) and np.all(np.isneginf(l_f[b]))
    for b in (1, 3, 4):
        for g in range(w.num_kv_heads):
            check_softmax(inp, o_s, l_s, o_f, l_f, sel, n_sel, b, g)
    # a launch bound below some row's n_sel flags that row with NaN
    o_b, l_b = run_softmax(inp, sel, n_sel, max_sel=3)
    for b in (1, 3, 4):
        over = int(n_sel[b].max()) > 3
        assert np.isnan(o_b[b]).all() == over
        assert np.isnan(l_b[b]).all() == over


def test_softmax_caller_page_list_any_order():
    # an explicit page list in any order: softmax is order-free
    w = small(121, batch=2, lens_range=None, top_k=6)
    inp = wl.make_inputs(w, device=DEV, lens=[1200, 640])
    s = cache_shape(inp)
    sel = torch.zeros((s.batch, s.num_kv_heads, s.max_pages_per_seq), dtype=torch.int32)
    n_sel = torch.zeros((s.batch, s.num_kv_heads), dtype=torch.int32)
    lists = {(0, 0): [74, 3, 0, 41], (0, 1): [5], (1, 0): [39, 38, 1], (1, 1): [0, 20, 10, 30]}
    for (b, g), pg in lists.items():
        sel[b, g, : len(pg)] = torch.tensor(pg, dtype=torch.int32)
        n_sel[b, g] = len(pg)
    sel, n_sel = sel.to(DEV), n_sel.to(DEV)
    o_s, l_s = run_softmax(inp, sel, n_sel, max_sel=4)
    o_f, l_f = run_softmax(inp)
    for (b, g) in lists:
        check_softmax(inp, o_s, l_s, o_f, l_f, sel, n_sel, b, g)


@pytest.mark.parametrize("seed", range(0, 64, 2))
def test_softmax_random_configurations(seed):
    # the random small configurations of the entmax sweep (every policy's
    # selection, dtypes, page sizes 1-64, ragged and empty rows): softmax over
    # each selection and over the full cache against the oracle on every pair
    from test_gpu_random import draw
    w, lens = draw(seed)
    print(f"[softmax random {seed}] {w}", flush=True)
    inp = wl.make_inputs(w, device=DEV, lens=lens)
    gpu = run_gpu(inp, w.policy)
    sel, n_sel = gpu.get("sel"), gpu.get("n_sel")
    max_sel = min(w.top_k, inp["max_pages"]) if w.policy == "topk" else 0
    o_s, l_s = run_softmax(inp, sel, n_sel, max_sel=max_sel)
    o_f, l_f = run_softmax(inp)
    for b in range(w.batch):
        if lens[b] == 0:
            assert np.all(o_s[b] == 0) and np.all(np.isneginf(l_f[b]))
            continue
        for g in range(w.num_kv_heads):
            check_softmax(inp, o_s, l_s, o_f, l_f, sel, n_sel, b, g)
