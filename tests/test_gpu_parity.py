"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases that the oracle finishes in seconds, spanning several workgroup
tiles and ragged tails, over every supported dtype / head_dim / group size /
page size and both selection policies, plus the degenerate cases of the
method.  Full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from oracle import pipeline
from sparse_kv_cache_page_amd import binding as B
from sparse_kv_cache_page_amd import workloads as wl

from gpu_util import cache_shape, check_pair, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(seed, **kw):
    base = dict(name="small", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                page_size=16, lens_range=(37, 1500), kv_dtype="bf16",
                q_std=2.0 / np.sqrt(128), scale=1.0, alpha=1.5, policy="topk", top_k=9,
                planted_per_kv_head=8, permute_pool=True, seed=seed)
    base.update(kw)
    return wl.Workload(**base)


def all_pairs(w):
    return [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]


def test_tiny_config_full_pipeline():
    w = wl.CONFIGS["tiny"]
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    ref = check_pair(inp, gpu, 0, 0, "topk")
    assert len(ref["sel"]) == 32


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (8, 2), (16, 2)])
def test_topk_shapes(kv_dtype, head_dim, heads):
    Hq, Hkv = heads
    w = small(11 + head_dim + Hq, kv_dtype=kv_dtype, head_dim=head_dim, num_q_heads=Hq,
              num_kv_heads=Hkv, q_std=2.0 / np.sqrt(head_dim))
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "topk")


@pytest.mark.parametrize("page_size", [1, 2, 8, 32, 64])
def test_topk_page_sizes(page_size):
    w = small(31 + page_size, page_size=page_size, lens_range=(5, 900),
              top_k=max(1, 150 // page_size))
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "topk")


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0, 1.1, 1.05, 1.02, 5.0, 8.0])
def test_alpha_values(alpha):
    w = small(41, alpha=alpha, planted_per_kv_head=4)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "topk")


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_dense_all_pages(alpha):
    w = small(51, alpha=alpha, lens_range=(200, 3000))
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "dense")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "dense")


def test_caller_page_list_out_of_range_entries():
    # entries outside [0, n_b) in a caller's list read nothing: the decode (with
    # and without page pruning) and the softmax path give the clean list's
    # results (the oracle checks the clean list)
    w = small(97, lens_range=(300, 1500))
    inp = wl.make_inputs(w, device=DEV)
    rng = np.random.default_rng(9)
    mp = inp["max_pages"]
    clean = np.full((w.batch, w.num_kv_heads, mp), -1, np.int32)
    dirty = np.full((w.batch, w.num_kv_heads, mp), -1, np.int32)
    nc = np.zeros((w.batch, w.num_kv_heads), np.int32)
    nd = np.zeros((w.batch, w.num_kv_heads), np.int32)
    lists = {}
    for b, g in all_pairs(w):
        n = inp["npages"][b]
        pick = sorted(rng.choice(n, size=int(rng.integers(1, n - 3)), replace=False).tolist())
        bad = [-5, n + 3, 1 << 30]
        mixed = list(pick)
        for x in bad:
            mixed.insert(int(rng.integers(0, len(mixed) + 1)), x)
        clean[b, g, :len(pick)] = pick
        dirty[b, g, :len(mixed)] = mixed
        nc[b, g], nd[b, g] = len(pick), len(mixed)
        lists[(b, g)] = pick
    t = lambda a: torch.tensor(a, device=DEV)
    for prune in (True, False):
        gc_ = run_gpu(inp, "topk", sel=t(clean), n_sel=t(nc), prune=prune)
        gd = run_gpu(inp, "topk", sel=t(dirty), n_sel=t(nd), prune=prune)
        for b, g in all_pairs(w):
            check_pair(inp, gc_, b, g, "topk", sel_override=lists[(b, g)])
        torch.testing.assert_close(gd["out"], gc_["out"], rtol=1e-6, atol=1e-7)
        torch.testing.assert_close(gd["tau"], gc_["tau"], rtol=1e-6, atol=1e-6)
        assert torch.equal(gd["n_support"], gc_["n_support"])
    s = cache_shape(inp)
    outs = []
    for sel_, n_ in ((clean, nc), (dirty, nd)):
        out = torch.empty_like(inp["q"])
        ws = torch.empty(max(B.softmax_workspace_bytes(s, mp), 256), dtype=torch.uint8,
                         device=DEV)
        B.softmax_decode(s, inp["q"], w.scale, inp["K"], inp["V"], inp["block_table"],
                         inp["seq_lens"], out, ws, sel=t(sel_), n_sel=t(n_), max_sel=mp)
        outs.append(out)
    torch.cuda.synchronize()
    torch.testing.assert_close(outs[1], outs[0], rtol=1e-6, atol=1e-7)


def test_caller_page_list():
    # decode over an explicit random page list (no selection stage)
    w = small(61, lens_range=(300, 2500))
    inp = wl.make_inputs(w, device=DEV)
    rng = np.random.default_rng(5)
    mp = inp["max_pages"]
    sel = np.full((w.batch, w.num_kv_heads, mp), -1, np.int32)
    nsel = np.zeros((w.batch, w.num_kv_heads), np.int32)
    lists = {}
    for b, g in all_pairs(w):
        n = inp["npages"][b]
        pick = sorted(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False).tolist())
        sel[b, g, :len(pick)] = pick
        nsel[b, g] = len(pick)
        lists[(b, g)] = pick
    gpu = run_gpu(inp, "topk", sel=torch.tensor(sel, device=DEV),
                  n_sel=torch.tensor(nsel, device=DEV))
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "topk", sel_override=lists[(b, g)])


@pytest.mark.parametrize("alpha,m16", [(2.0, False), (1.5, False), (1.25, False), (1.5, True)])
def test_gauss_policy(alpha, m16):
    w = small(71, alpha=alpha, policy="gauss", clusters=16, planted_per_kv_head=0,
              lens_range=(100, 1200), delta=0.1, moments_bf16=m16)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "gauss")


def test_gauss_guard_keeps_argmax():
    # every page holds 8 zero keys and 8 copies of e_0, so u = m + sigma exactly
    # for every head; with ~40 such pages per row the Gaussian estimate tau-hat
    # lies above every (alpha-1) u and nothing clears the bar: the guard keeps
    # the largest bound, and since all bounds tie, page 0
    w = small(81, alpha=2.0, policy="gauss", planted_per_kv_head=0, lens_range=(600, 700),
              delta=0.0)
    inp = wl.make_inputs(w, device=DEV)
    K = inp["K"]
    K.zero_()
    K[:, :, 8:, 0] = 1.0
    # |q_0| must be large enough that F(u) > 1 for every head, i.e. tau-hat > u:
    # with q_0 = 0.5, sigma = 0.25 and F(m + sigma) = 16 * 40 * sigma * I_1(-1) ~ 13
    inp["q"][:, :, 0] = 0.5
    gpu = run_gpu(inp, "gauss")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "gauss")
        assert int(gpu["n_sel"][b, g]) == 1 and int(gpu["sel"][b, g, 0]) == 0


@pytest.mark.parametrize("alpha,page_size,m16", [(2.0, 16, False), (1.5, 8, False),
                                                 (1.25, 32, False), (4.0 / 3.0, 64, False),
                                                 (2.0, 16, True)])
def test_gauss_est_policy(alpha, page_size, m16):
    # expected-maximum estimate m + e_n sqrt(v): e_P on full pages, e_n on the
    # ragged last page of each row
    w = small(73, alpha=alpha, policy="gauss_est", clusters=16, planted_per_kv_head=0,
              page_size=page_size, lens_range=(100, 1200), delta=0.1, moments_bf16=m16)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_est")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "gauss_est")


@pytest.mark.parametrize("m16", [False, True])
@pytest.mark.parametrize("alpha,page_size,eps", [(2.0, 16, 1e-4), (1.5, 8, 1e-3),
                                                 (1.25, 32, 1e-2), (4.0 / 3.0, 64, 3e-4)])
def test_gauss_mass_policy(alpha, page_size, eps, m16):
    # expected page mass n_p E[(X - tau_hat)_+^gamma] against eps (ragged last
    # pages use their own token counts)
    # (m16: the compact metadata format, bf16 page mean / variance)
    w = small(77, alpha=alpha, policy="gauss_mass", clusters=16, planted_per_kv_head=0,
              page_size=page_size, lens_range=(100, 1200), delta=eps, moments_bf16=m16)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_mass")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "gauss_mass")


def test_gauss_mass_guard_keeps_argmax():
    # no page can hold a mass above 1: eps = 1.5 leaves only the guard's page
    w = small(83, alpha=2.0, policy="gauss_mass", clusters=16, planted_per_kv_head=0,
              lens_range=(300, 900), delta=1.5)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_mass")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "gauss_mass")
        assert int(gpu["n_sel"][b, g]) == 1


def test_gauss_est_guard_keeps_argmax():
    # the guard case of the box-bound reading, with tau-hat also above
    # m + e_16 sigma: F(m + e_16 sigma) = 16 * 40 * sigma * I_1(-e_16) ~ 2.5 > 1
    w = small(81, alpha=2.0, policy="gauss_est", planted_per_kv_head=0,
              lens_range=(600, 700), delta=0.0)
    inp = wl.make_inputs(w, device=DEV)
    K = inp["K"]
    K.zero_()
    K[:, :, 8:, 0] = 1.0
    inp["q"][:, :, 0] = 0.5
    gpu = run_gpu(inp, "gauss_est")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "gauss_est")
        assert int(gpu["n_sel"][b, g]) == 1 and int(gpu["sel"][b, g, 0]) == 0


@pytest.mark.parametrize("policy,alpha", [("gauss", 2.0), ("gauss_est", 1.5), ("gauss_mass", 2.0)])
def test_gauss_long_rows(policy, alpha):
    # pages of 2 tokens, rows of 4500-6000 pages: the tau-hat kernel's variant
    # that reads the moments from global memory (> 4096 pages) and the marking
    # kernel's compaction over several 4096-page chunks
    w = small(161, page_size=2, lens_range=(9000, 12000), num_q_heads=4, num_kv_heads=2,
              head_dim=64, q_std=2.0 / 8.0, alpha=alpha, policy=policy, clusters=16,
              planted_per_kv_head=0, delta=1e-5 if policy == "gauss_mass" else 0.1, batch=2)
    inp = wl.make_inputs(w, device=DEV)
    assert min(inp["npages"]) > 4096
    gpu = run_gpu(inp, policy)
    for b, g in [(0, 0), (1, 1)]:
        check_pair(inp, gpu, b, g, policy)


def _skipped_pages(gpu, w, alpha):
    # the decode's pruning rule, replayed on the host in fp32
    a1 = np.float32(alpha - 1.0)
    ub = gpu["ub"].cpu().numpy()
    zlb = gpu["zlb"].cpu().numpy()
    sel = gpu["sel"].cpu().numpy()
    nsel = gpu["n_sel"].cpu().numpy()
    G = w.group
    skipped = total = 0
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            for p in sel[b, g, :nsel[b, g]]:
                below = True
                for h in range(g * G, (g + 1) * G):
                    x = a1 * ub[b, g, p, h - g * G]
                    s1 = np.float32(1e-3) * (np.float32(1) + abs(x))
                    s2 = np.float32(1e-4) * (np.float32(1) + abs(zlb[b, h]))
                    below &= bool(x + s1 < zlb[b, h] - np.float32(1) - s2)
                skipped += below
                total += 1
    return skipped, total


@pytest.mark.parametrize("case", ["planted", "random", "dense", "fused"])
def test_page_pruning_is_exact(case):
    # with per-head bounds the decode skips the selected pages that cannot hold
    # any head's support; tau, the output and the support sizes must be those
    # of the unpruned decode, bit for bit
    w = small(171, lens_range=(2000, 6000), top_k=200,
              planted_per_kv_head=0 if case == "random" else 8)
    inp = wl.make_inputs(w, device=DEV)
    pol = "dense" if case == "dense" else "topk"
    if case == "fused":
        s = cache_shape(inp)
        ref = run_gpu(inp, pol, prune=False)
        outs = []
        for ub, zlb in [(None, None), (ref["ub"], torch.empty_like(ref["tau"]))]:
            ws = torch.zeros(B.decode_fused_workspace_bytes(s, w.top_k), dtype=torch.uint8,
                             device=DEV)
            o = torch.empty_like(ref["out"])
            t = torch.empty_like(ref["tau"])
            B.entmax_decode(s, inp["q"], w.scale, w.alpha, inp["K"], inp["V"],
                            inp["block_table"], inp["seq_lens"], o, ws, sel=ref["sel"],
                            n_sel=ref["n_sel"], max_sel=w.top_k, tau=t, fused=True, ub=ub,
                            zlb=zlb)
            outs.append((o, t))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
        return
    plain = run_gpu(inp, pol, prune=False)
    pruned = run_gpu(inp, pol, prune=True)
    for k in ("out", "tau", "n_support"):
        assert torch.equal(plain[k], pruned[k]), k
    if case == "planted":
        skipped, total = _skipped_pages(pruned, w, w.alpha)
        assert skipped > 0.8 * total, (skipped, total)
    for b, g in [(0, 0), (w.batch - 1, 1)]:
        check_pair(inp, pruned, b, g, pol)


@pytest.mark.parametrize("kw", [
    dict(num_q_heads=16, num_kv_heads=2), dict(num_q_heads=4, num_kv_heads=4),
    dict(kv_dtype="f32", head_dim=64, q_std=2.0 / 8.0), dict(page_size=64, top_k=40),
    dict(page_size=1, lens_range=(300, 3000), top_k=600), dict(alpha=1.25), dict(alpha=2.0),
    dict(alpha=3.0, q_std=4.0 / np.sqrt(128)),
])
def test_page_pruning_is_exact_shapes(kw):
    # the pruned decode equals the unpruned one bit for bit across group sizes,
    # dtypes, head dims, page sizes and alpha (planted keys, so pages get pruned)
    base = dict(lens_range=(2000, 6000), top_k=200, planted_per_kv_head=8)
    base.update(kw)
    w = small(181 + len(kw) + int(10 * base.get("alpha", 0)), **base)
    inp = wl.make_inputs(w, device=DEV)
    plain = run_gpu(inp, "topk", prune=False)
    pruned = run_gpu(inp, "topk", prune=True)
    for k in ("out", "tau", "n_support"):
        assert torch.equal(plain[k], pruned[k]), k
    skipped, total = _skipped_pages(pruned, w, w.alpha)
    print(f"pruned {skipped} of {total} selected pages")
    check_pair(inp, pruned, w.batch - 1, w.num_kv_heads - 1, "topk")


@pytest.mark.parametrize("policy", ["gauss", "gauss_est", "gauss_mass"])
def test_page_pruning_is_exact_gaussian(policy):
    # pruning over the Gaussian policies' selections (clustered keys, alpha 2)
    w = small(191, lens_range=(1500, 4000), alpha=2.0, policy=policy,
              delta=1e-4 if policy == "gauss_mass" else 0.1,
              planted_per_kv_head=0, clusters=64, cluster_sigma=0.5)
    inp = wl.make_inputs(w, device=DEV)
    plain = run_gpu(inp, policy, prune=False)
    pruned = run_gpu(inp, policy, prune=True)
    for k in ("sel", "n_sel", "out", "tau", "n_support"):
        assert torch.equal(plain[k], pruned[k]), k
    skipped, total = _skipped_pages(pruned, w, w.alpha)
    print(f"{policy}: pruned {skipped} of {total} selected pages")
    check_pair(inp, pruned, 0, 0, policy)


def test_edge_single_token_rows():
    w = small(91, lens_range=None, seq_len=1, batch=2, top_k=3)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    for b, g in all_pairs(w):
        check_pair(inp, gpu, b, g, "topk")
        assert float(gpu["tau"][b, 0]) == pytest.approx(
            float(0.5 * w.scale * (pipeline.widen(inp["q"][b, 0]) @
                                   pipeline.widen(inp["K"][inp["block_table"][b, 0].long(), 0, 0])) - 1),
            abs=1e-5)


def test_edge_topk_covers_all_and_one():
    for k in (1, 10_000):
        w = small(101 + k, top_k=k)
        inp = wl.make_inputs(w, device=DEV)
        gpu = run_gpu(inp, "topk")
        for b, g in all_pairs(w):
            check_pair(inp, gpu, b, g, "topk")
            n = inp["npages"][b]
            assert int(gpu["n_sel"][b, g]) == min(k, n)


def test_edge_ties_shared_pages_constant_keys():
    # rows 0 and 1 share every physical page and the query; page 5 carries a
    # planted key and is copied onto pages 0, 3, 6, ... so 15 pages tie for the
    # largest bound (the tie rule, lowest index, decides the top-7); page 7
    # holds one constant key (zero variance) for the Gaussian branch
    for pol in ("topk", "gauss"):
        w = small(111, batch=2, lens_range=None, seq_len=16 * 40, permute_pool=False,
                  planted_per_kv_head=0, top_k=7, policy=pol)
        inp = wl.make_inputs(w, device=DEV)
        bt = inp["block_table"].clone()
        bt[1] = bt[0]
        inp["block_table"] = bt
        q = inp["q"]
        q[1] = q[0]
        K = inp["K"]
        G = w.group
        src = int(bt[0, 5])
        for g in range(w.num_kv_heads):
            K[src, g, 0] = (3.0 * q[0, g * G] / w.q_std).to(K.dtype)
        for p in range(0, 40, 3):
            K[int(bt[0, p])] = K[src]
        c = int(bt[0, 7])
        K[c] = K[c][:, :1, :].expand(-1, w.page_size, -1).clone()
        gpu = run_gpu(inp, pol)
        for b, g in all_pairs(w):
            check_pair(inp, gpu, b, g, pol)
        assert torch.equal(gpu["sel"][0], gpu["sel"][1])
        assert torch.equal(gpu["out"][0], gpu["out"][1])
        if pol == "topk":
            assert gpu["sel"][0, 0, :7].tolist() == [0, 3, 5, 6, 9, 12, 15]


def test_max_sel_too_small_flags_nan():
    w = small(121, top_k=20, lens_range=(400, 900))
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    s = B.CacheShape(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                     inp["max_pages"], inp["num_phys_pages"], torch.bfloat16)
    out = torch.zeros_like(gpu["out"])
    ws = torch.empty(B.decode_workspace_bytes(s, 5), dtype=torch.uint8, device=DEV)
    B.entmax_decode(s, inp["q"], w.scale, w.alpha, inp["K"], inp["V"], inp["block_table"],
                    inp["seq_lens"], out, ws, sel=gpu["sel"], n_sel=gpu["n_sel"], max_sel=5)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


def test_refresh_last_page_matches_full_build():
    # append tokens to every row, refresh only the last page, compare with a
    # from-scratch build
    w = small(131, lens_range=(40, 700), planted_per_kv_head=0)
    inp = wl.make_inputs(w, device=DEV)
    s = B.CacheShape(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                     inp["max_pages"], inp["num_phys_pages"], torch.bfloat16)
    lens = torch.tensor([L - 3 for L in inp["lens"]], dtype=torch.int32, device=DEV)
    mk = lambda: [torch.zeros(s.num_phys_pages, s.num_kv_heads, s.head_dim, dtype=t, device=DEV)
                  for t in (torch.bfloat16, torch.bfloat16, torch.float32, torch.float32)]
    a = mk()
    B.build_page_meta(s, inp["K"], inp["block_table"], lens, *a)
    # three decode steps append one token each; refresh the page holding it
    P = w.page_size
    for _ in range(3):
        lens += 1
        last = ((lens + P - 1) // P - 1).to(torch.int32)
        B.build_page_meta(s, inp["K"], inp["block_table"], lens, *a, first_page=last, span=1)
    b_ = mk()
    B.build_page_meta(s, inp["K"], inp["block_table"], lens, *b_)
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        assert torch.equal(x, y)


def test_deterministic_repeat():
    w = small(141, lens_range=(500, 2000))
    inp = wl.make_inputs(w, device=DEV)
    g1 = run_gpu(inp, "topk")
    g2 = run_gpu(inp, "topk")
    for k in ("ubg", "sel", "n_sel", "out", "tau"):
        # entries past a row's pages are never written (NaN / sentinel in both)
        assert torch.equal(torch.nan_to_num(g1[k], nan=-1.0), torch.nan_to_num(g2[k], nan=-1.0)), k


@pytest.mark.parametrize("lens", [(2100, 4000), (5000, 9000), (16500, 17500)])
def test_topk_long_rows(lens):
    # page size 1 gives rows of thousands of pages: the wave select (<= 4096
    # pages), the block select with LDS keys (<= 16384) and with keys in L2
    w = small(151, page_size=1, lens_range=lens, num_q_heads=4, num_kv_heads=2,
              head_dim=64, q_std=2.0 / 8.0, top_k=700, planted_per_kv_head=4)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    for b, g in [(0, 0), (w.batch - 1, 1)]:
        check_pair(inp, gpu, b, g, "topk")


@pytest.mark.parametrize("lens", [[12000, 9000], [12001, 9000], [40000, 33000],
                                  [40001, 33000]])
def test_topk_long_row_widths(lens):
    # the 1024-thread select with 16 and 64 keys per thread, its bounds read
    # with 16-byte loads when the row width is a multiple of 4 and one load per
    # key otherwise
    w = small(157, page_size=1, lens_range=None, batch=2, num_q_heads=4, num_kv_heads=2,
              head_dim=64, q_std=2.0 / 8.0, top_k=700, planted_per_kv_head=4)
    inp = wl.make_inputs(w, device=DEV, lens=lens)
    print(f"[parity] long-row widths {lens}", flush=True)
    gpu = run_gpu(inp, "topk")
    for b, g in [(0, 0), (1, 1)]:
        check_pair(inp, gpu, b, g, "topk")


def test_pruning_probe_long_selection():
    # more than 8192 selected pages: the pruning probe walks the selection in
    # two rounds of 32 slots per thread
    w = small(163, page_size=1, lens_range=None, batch=2, num_q_heads=4, num_kv_heads=2,
              head_dim=64, q_std=2.0 / 8.0, top_k=9000, planted_per_kv_head=4)
    inp = wl.make_inputs(w, device=DEV, lens=[20000, 9500])
    print("[parity] pruning probe over 9000 selected pages", flush=True)
    gpu = run_gpu(inp, "topk", prune=True)
    for b, g in [(0, 0), (0, 1), (1, 1)]:
        check_pair(inp, gpu, b, g, "topk")


@pytest.mark.parametrize("policy,prune", [("topk", True), ("topk", False), ("gauss", False),
                                          ("gauss_est", True), ("gauss_mass", False),
                                          ("dense", False)])
def test_edge_empty_rows(policy, prune):
    # idle batch slots (seq_len 0) next to rows with tokens: the empty rows get
    # n_sel = 0, a zero output, tau NaN and support 0; the other rows are those
    # of the oracle
    gauss = policy in ("gauss", "gauss_est", "gauss_mass")
    w = small(211, batch=5, lens_range=None, alpha=2.0 if gauss else 1.5, policy=policy,
              delta=1e-3 if policy == "gauss_mass" else 0.1,
              planted_per_kv_head=0 if gauss else 8, clusters=64 if gauss else 0)
    inp = wl.make_inputs(w, device=DEV, lens=[0, 700, 0, 33, 1500])
    gpu = run_gpu(inp, policy, prune=prune)
    G = w.group
    for b in (0, 2):
        for g in range(w.num_kv_heads):
            if policy != "dense":
                assert int(gpu["n_sel"][b, g]) == 0
        assert torch.equal(gpu["out"][b], torch.zeros_like(gpu["out"][b]))
        assert torch.isnan(gpu["tau"][b]).all()
        assert int(gpu["n_support"][b].abs().sum()) == 0
        if gauss:
            assert torch.isnan(gpu["tau_hat"][b]).all()
    for b in (1, 3, 4):
        for g in range(w.num_kv_heads):
            check_pair(inp, gpu, b, g, policy)


def test_edge_empty_rows_fused_paths():
    # the fused step and the fused decode on a batch with idle slots
    from sparse_kv_cache_page_amd.engine import PagedEntmaxDecoder
    w = small(221, batch=4, lens_range=None, top_k=20)
    inp = wl.make_inputs(w, device=DEV, lens=[900, 0, 2000, 0])
    s = cache_shape(inp)
    f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale,
                           fused=True)
    f.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
    f.out.fill_(float("nan"))
    f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    ws = torch.zeros(B.decode_fused_workspace_bytes(s, w.top_k), dtype=torch.uint8, device=DEV)
    out2 = torch.full_like(f.out, float("nan"))
    tau2 = torch.full_like(f.tau, 0.0)
    sup2 = torch.full_like(f.n_support, 7)
    torch.cuda.synchronize()
    B.entmax_decode(s, inp["q"], w.scale, w.alpha, inp["K"], inp["V"], inp["block_table"],
                    inp["seq_lens"], out2, ws, sel=f.sel, n_sel=f.n_sel, max_sel=w.top_k,
                    tau=tau2, n_support=sup2, fused=True)
    torch.cuda.synchronize()
    for out, tau, sup in ((f.out, f.tau, f.n_support), (out2, tau2, sup2)):
        for b in (1, 3):
            assert torch.equal(out[b], torch.zeros_like(out[b]))
            assert torch.isnan(tau[b]).all()
            assert int(sup[b].abs().sum()) == 0
        assert not torch.isnan(out[0]).any() and not torch.isnan(out[2]).any()
    assert int(f.n_sel[1].abs().sum()) == 0 and int(f.n_sel[3].abs().sum()) == 0
    gpu = dict(kmin=f.kmin, kmax=f.kmax, ubg=f.ubg, sel=f.sel, n_sel=f.n_sel, out=f.out,
               tau=f.tau)
    for b, g in [(0, 0), (2, 1)]:
        check_pair(inp, gpu, b, g, "topk", check_meta=False)


def test_validate_cache_counts_planted_errors():
    # device-side check of seq_lens and the block table: valid inputs give
    # (0, 0); planted bad lengths and out-of-pool pages are counted, slots past
    # a row's pages are not looked at
    w = small(231, batch=5, lens_range=None)
    inp = wl.make_inputs(w, device=DEV, lens=[900, 0, 2000, 40, 333])
    s = cache_shape(inp)
    assert B.validate_cache(s, inp["block_table"], inp["seq_lens"]) == (0, 0)
    bt = inp["block_table"].clone()
    lens = inp["seq_lens"].clone()
    P, mp = w.page_size, inp["max_pages"]
    lens[1] = mp * P + 1            # too long
    lens[4] = -3                    # negative
    bt[0, 0] = s.num_phys_pages     # outside the pool
    bt[3, 2] = -1                   # row 3 has 3 pages: its last one
    bt[2, mp - 1] = 12345678        # row 2 (2000 tokens) ends before this slot if mp > 125
    expect_bt = 2 + (1 if (2000 + P - 1) // P == mp else 0)
    assert B.validate_cache(s, bt, lens) == (2, expect_bt)
    lens[1] = mp * P                # exactly full is valid
    assert B.validate_cache(s, bt, lens)[0] == 1
