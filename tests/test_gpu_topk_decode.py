"""GPU tests of ekv_topk_decode (top-k selection inside the decode's key launch).

Each work item selects its pair's pages itself, probes the heads' best pages
for the pruning bound and scores an even share of the pages left to read; the
results must be bit-identical to ekv_select_pages(TOPK) followed by the pruned
(or unpruned) ekv_entmax_decode on the same bounds, whichever of its two
paths the shape takes (the fused selection up to 1024 selected pages and 8192
pages per row, the separate kernels beyond), and match the oracle on sampled
pairs.
"""
import numpy as np
import pytest
import torch

from sparse_kv_cache_page_amd import binding as B
from sparse_kv_cache_page_amd import workloads as wl
from sparse_kv_cache_page_amd.engine import PagedEntmaxDecoder

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


def both(inp, prune, hinted=False):
    """(separate select + decode, topk_decode) decoders after one step each; with
    hinted, the second one scores through ekv_score_box_pages and passes its
    best-page hints to ekv_topk_decode."""
    w = inp["workload"]
    s = cache_shape(inp)
    a = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale,
                           prune=prune)
    f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale,
                           prune=prune)
    for d in (a, f):
        d.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
    a.score(inp["q"], inp["block_table"], inp["seq_lens"])
    if hinted:
        f.score_box(inp["q"], inp["block_table"], inp["seq_lens"])
    else:
        f.score(inp["q"], inp["block_table"], inp["seq_lens"])
    a.select(inp["seq_lens"])
    a.decode(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    f.sel.fill_(-7)
    f.out.fill_(float("nan"))
    f.topk_decode(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"],
                  use_hint=hinted)
    torch.cuda.synchronize()
    return a, f


def bits(x):
    # bit patterns, so NaN entries (empty rows) compare equal to themselves
    return x.contiguous().view(torch.int32)


def assert_same(a, f, inp):
    w = inp["workload"]
    assert torch.equal(a.n_sel, f.n_sel)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            n = int(a.n_sel[b, g])
            assert torch.equal(a.sel[b, g, :n], f.sel[b, g, :n]), f"sel b{b} g{g}"
    assert torch.equal(bits(a.out), bits(f.out))
    assert torch.equal(bits(a.tau), bits(f.tau))
    assert torch.equal(a.n_support, f.n_support)


CASES = [
    dict(), dict(num_q_heads=16, num_kv_heads=2), dict(num_q_heads=4, num_kv_heads=4),
    dict(num_q_heads=4, num_kv_heads=2), dict(kv_dtype="f32", head_dim=64, q_std=2.0 / 8.0),
    dict(head_dim=64, q_std=0.25), dict(page_size=32, top_k=5), dict(page_size=64, top_k=3),
    dict(page_size=1, lens_range=(3, 300), top_k=40), dict(top_k=1000),
    dict(page_size=1, lens_range=(3000, 6000), top_k=500, head_dim=64, q_std=0.25),
    # beyond the fused selection's limits: the separate kernels
    dict(page_size=1, lens_range=(1500, 3000), top_k=1500),
    dict(page_size=1, lens_range=(9000, 9500), top_k=200, batch=2),
    # one token per row, and k = 1
    dict(lens_range=(1, 1), top_k=4), dict(top_k=1),
]


@pytest.mark.parametrize("mode", ["prune", "hinted", "plain"])
@pytest.mark.parametrize("kw", CASES)
def test_topk_decode_matches_separate(kw, mode):
    w = small(301 + len(kw) + 7 * sum(len(str(v)) for v in kw.values()), **kw)
    inp = wl.make_inputs(w, device=DEV)
    print(f"[topk_decode] {kw} {mode}", flush=True)
    a, f = both(inp, mode != "plain", hinted=mode == "hinted")
    assert_same(a, f, inp)
    if mode == "hinted":
        # the box-only scorer writes the bounds ekv_score_pages writes
        m = inp["npages"]
        for b in range(w.batch):
            assert torch.equal(a.ubg[b, :, :m[b]], f.ubg[b, :, :m[b]])
            assert torch.equal(a.ub[b, :, :m[b]], f.ub[b, :, :m[b]])


def test_topk_decode_empty_rows():
    # idle batch slots (seq_len 0) next to full rows
    w = small(377, batch=4, lens_range=None, top_k=7)
    inp = wl.make_inputs(w, device=DEV, lens=[850, 0, 230, 0])
    a, f = both(inp, True, hinted=True)
    assert_same(a, f, inp)
    assert int(f.n_sel[1, 0]) == 0 and int(f.n_sel[3, 1]) == 0
    assert bool((f.out[1] == 0).all()) and bool(torch.isnan(f.tau[1]).all())


@pytest.mark.parametrize("lens", [[3000, 4000], [3001, 4001], [6000, 8000], [6003, 8001]])
def test_topk_decode_long_row_layouts(lens):
    # 16 and 32 pages per thread (rows of up to 4096 and 8192 pages), with the
    # block-table width a multiple of 4 (the bounds and block-table rows are
    # read coalesced and handed out through LDS) or not (per-thread loads)
    w = small(433, lens_range=None, page_size=1, top_k=300, batch=2, head_dim=64,
              q_std=0.25)
    inp = wl.make_inputs(w, device=DEV, lens=lens)
    assert inp["max_pages"] == max(lens)
    print(f"[topk_decode] long-row layout {lens}", flush=True)
    a, f = both(inp, True, hinted=True)
    assert_same(a, f, inp)


@pytest.mark.parametrize("fill", ["random", "other_cache"])
def test_topk_decode_foreign_hints(fill):
    # hints that this call's scorer did not write (random bytes, or another
    # cache's hints for the same shape): the probe reads a hinted physical page
    # only inside the pool and uses it only where the block table agrees, so
    # the results still equal the separate path's
    lens = [1500, 700, 37]
    w = small(411, lens_range=None)
    inp = wl.make_inputs(w, device=DEV, lens=lens)
    a, f = both(inp, True, hinted=True)
    if fill == "random":
        g = torch.Generator(device="cpu").manual_seed(5)
        f.hint.copy_(torch.randint(0, 256, f.hint.shape, dtype=torch.uint8, generator=g))
    else:
        inp2 = wl.make_inputs(small(412, lens_range=None), device=DEV, lens=lens)
        assert inp2["num_phys_pages"] == inp["num_phys_pages"]
        assert not torch.equal(inp2["block_table"], inp["block_table"])
        o = PagedEntmaxDecoder(cache_shape(inp2), policy="topk", top_k=w.top_k, alpha=w.alpha,
                               scale=w.scale)
        o.build_meta(inp2["K"], inp2["block_table"], inp2["seq_lens"])
        o.score_box(inp2["q"], inp2["block_table"], inp2["seq_lens"])
        f.hint.copy_(o.hint)
    print(f"[topk_decode] foreign hints: {fill}", flush=True)
    f.sel.fill_(-7)
    f.out.fill_(float("nan"))
    f.topk_decode(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"],
                  use_hint=True)
    torch.cuda.synchronize()
    assert_same(a, f, inp)


@pytest.mark.parametrize("kw", [dict(), dict(num_q_heads=16, num_kv_heads=2, page_size=32)])
def test_topk_decode_against_oracle(kw):
    w = small(391, **kw)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "topk")
    s = cache_shape(inp)
    f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale)
    f.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
    f.score(inp["q"], inp["block_table"], inp["seq_lens"])
    f.topk_decode(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    torch.cuda.synchronize()
    gpu.update(sel=f.sel, n_sel=f.n_sel, out=f.out, tau=f.tau)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            check_pair(inp, gpu, b, g, "topk")


def test_topk_decode_graph_replays():
    w = small(399, batch=4, lens_range=(500, 3000), top_k=40)
    inp = wl.make_inputs(w, device=DEV)
    a, f = both(inp, True)
    ref = f.out.clone()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        f.topk_decode(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        f.topk_decode(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    for _ in range(3):
        f.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f.out, ref)
        assert_same(a, f, inp)


def test_topk_decode_workspace_and_errors():
    w = small(401)
    inp = wl.make_inputs(w, device=DEV)
    s = cache_shape(inp)
    need = B.topk_decode_workspace_bytes(s, w.top_k)
    assert need >= B.decode_workspace_bytes(s, w.top_k)
    f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale)
    small_ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.EkvError):
        B.topk_decode(s, inp["q"], w.scale, w.alpha, inp["K"], inp["V"], inp["block_table"],
                      inp["seq_lens"], w.top_k, f.ubg, f.sel, f.n_sel, f.out, small_ws)
    with pytest.raises(B.EkvError):
        B.topk_decode(s, inp["q"], w.scale, 1.0, inp["K"], inp["V"], inp["block_table"],
                      inp["seq_lens"], w.top_k, f.ubg, f.sel, f.n_sel, f.out, f.ws)
