"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (PagedEntmaxDecoder), on sampled (row, KV head) pairs that the
oracle recomputes one by one, plus properties checked on every pair.

Workloads (seeded, synthetic; see sparse_kv_cache_page_amd/workloads.py):
  gqa     B8, 32q/8kv, d128, L 32768, P16, bf16, alpha 1.5, top-256
  gauss   gqa shapes, clustered keys, alpha 2, Gaussian-aware, delta 0.1
  ragged  B64, L ~ U[4096, 65536], permuted pool, alpha 1.5, top-512
  stress  B32, 64q/8kv, L 131072, P32, alpha in {1.25, 1.5, 2},
          top-512 / top-128 / Gaussian / dense, query temperature sets the
          support size (about 16 to 4096 tokens)
"""
import math

import pytest
import torch

from sparse_kv_cache_page_amd import binding as B
from sparse_kv_cache_page_amd import workloads as wl
from sparse_kv_cache_page_amd.engine import PagedEntmaxDecoder

from gpu_util import cache_shape, check_pair, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def check_properties(inp, gpu, policy, top_k):
    """Selection well-formed and outputs finite on every pair."""
    w = inp["workload"]
    lens = torch.tensor(inp["npages"], device=DEV)
    if policy != "dense":
        n_sel = gpu["n_sel"]
        if policy == "topk":
            assert torch.equal(n_sel, torch.minimum(lens, torch.tensor(top_k, device=DEV))[:, None]
                               .expand_as(n_sel).to(n_sel.dtype))
        assert bool((n_sel >= 1).all())
        sel = gpu["sel"].cpu()
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                s = sel[b, g, :int(n_sel[b, g])]
                assert bool((s[1:] > s[:-1]).all()) and int(s[0]) >= 0
                assert int(s[-1]) < inp["npages"][b]
    assert bool(torch.isfinite(gpu["out"]).all())
    assert bool(torch.isfinite(gpu["tau"]).all())


def decoder_matches(inp, gpu, policy, alpha, top_k, delta, scale, q):
    """The benchmark's call sequence gives bit-identical results.

    For the top-k policy that is ekv_score_pages followed by ekv_topk_decode
    (top-k selection inside the decode's key launch, page pruning), exactly
    as bench.py's Layer issues them; ekv_decode_step (the same two calls
    behind one entry point) is checked too.  Every output must equal the
    separate score / select / decode calls of `gpu`, which the oracle checked.
    """
    s = cache_shape(inp)
    fused = policy == "topk"
    dec = PagedEntmaxDecoder(s, policy=policy, top_k=top_k, alpha=alpha, scale=scale,
                             delta=delta, fused=fused)
    dec.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
    if fused:
        dec.score(q, inp["block_table"], inp["seq_lens"])
        dec.topk_decode(q, inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    else:
        dec.step(q, inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    torch.cuda.synchronize()
    assert torch.equal(dec.out, gpu["out"]) and torch.equal(dec.tau, gpu["tau"])
    assert torch.equal(dec.n_support, gpu["n_support"])
    if policy != "dense":
        assert torch.equal(dec.n_sel, gpu["n_sel"])
        for b in range(s.batch):
            for g in range(s.num_kv_heads):
                n = int(gpu["n_sel"][b, g])
                assert torch.equal(dec.sel[b, g, :n], gpu["sel"][b, g, :n]), f"sel b{b} g{g}"
        npg = torch.tensor(inp["npages"], device=DEV)
        live = torch.arange(s.max_pages_per_seq, device=DEV)[None, :] < npg[:, None]
        live = live[:, None, :].expand_as(gpu["ubg"])
        assert torch.equal(dec.ubg[live], gpu["ubg"][live])
    if fused:
        out1, tau1 = dec.out.clone(), dec.tau.clone()
        ns1 = dec.n_support.clone()
        dec.out.fill_(float("nan"))
        dec.fused_step(q, inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
        torch.cuda.synchronize()
        assert torch.equal(dec.out, out1) and torch.equal(dec.tau, tau1)
        assert torch.equal(dec.n_support, ns1)
    return dec


@pytest.mark.parametrize("name,pairs", [
    ("gqa", [(0, 0), (3, 5), (7, 7)]),
    ("gauss", [(0, 0), (5, 3)]),
    ("ragged", [(0, 0), (17, 4), (63, 7)]),
])
def test_fullsize_config(name, pairs):
    w = wl.CONFIGS[name]
    print(f"[fullsize] {name}: generating", flush=True)
    inp = wl.make_inputs(w, device=DEV)
    pol = w.policy
    gpu = run_gpu(inp, pol)
    check_properties(inp, gpu, pol, w.top_k)
    for b, g in pairs:
        print(f"[fullsize] {name}: oracle pair b{b} g{g}", flush=True)
        check_pair(inp, gpu, b, g, pol)
    decoder_matches(inp, gpu, pol, w.alpha, w.top_k, w.delta, w.scale, inp["q"])


def test_fullsize_gauss_est():
    # gauss shapes with the expected-maximum estimate of a page's maximum score
    w = wl.variant("gauss", policy="gauss_est")
    print("[fullsize] gauss_est: generating", flush=True)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_est")
    check_properties(inp, gpu, "gauss_est", w.top_k)
    for b, g in [(0, 0), (6, 2)]:
        print(f"[fullsize] gauss_est: oracle pair b{b} g{g}", flush=True)
        check_pair(inp, gpu, b, g, "gauss_est")
    decoder_matches(inp, gpu, "gauss_est", w.alpha, w.top_k, w.delta, w.scale, inp["q"])


def test_fullsize_gauss_mass():
    # gauss shapes with the expected-mass rule (mass threshold 1e-4)
    w = wl.CONFIGS["gauss_mass"]
    print("[fullsize] gauss_mass: generating", flush=True)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_mass")
    check_properties(inp, gpu, "gauss_mass", w.top_k)
    for b, g in [(0, 0), (6, 2)]:
        print(f"[fullsize] gauss_mass: oracle pair b{b} g{g}", flush=True)
        check_pair(inp, gpu, b, g, "gauss_mass")
    decoder_matches(inp, gpu, "gauss_mass", w.alpha, w.top_k, w.delta, w.scale, inp["q"])


def test_fullsize_gauss_mass_compact_moments():
    # the expected-mass rule on bf16 page moments (the compact metadata format)
    w = wl.CONFIGS["gauss_mass_m16"]
    print("[fullsize] gauss_mass_m16: generating", flush=True)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_mass")
    check_properties(inp, gpu, "gauss_mass", w.top_k)
    for b, g in [(1, 1), (7, 6)]:
        print(f"[fullsize] gauss_mass_m16: oracle pair b{b} g{g}", flush=True)
        check_pair(inp, gpu, b, g, "gauss_mass")


@pytest.fixture(scope="module")
def stress_inputs():
    w = wl.CONFIGS["stress"]
    print("[fullsize] stress: generating 16 GiB of K/V", flush=True)
    inp = wl.make_inputs(w, device=DEV)
    yield inp
    del inp
    torch.cuda.empty_cache()


STRESS_CASES = [
    (1.25, 0, "topk", 512), (1.25, 1, "topk", 128), (1.25, 2, "dense", 0),
    (1.5, 0, "gauss", 0), (1.5, 1, "topk", 512), (1.5, 2, "topk", 128),
    (2.0, 0, "dense", 0), (2.0, 1, "gauss", 0), (2.0, 2, "topk", 512),
    (1.25, 1, "gauss_est", 0),
]


@pytest.mark.parametrize("alpha,ti,policy,top_k", STRESS_CASES)
def test_fullsize_stress(stress_inputs, alpha, ti, policy, top_k):
    inp = stress_inputs
    w = wl.variant("stress", alpha=alpha, policy=policy, top_k=top_k or 512, delta=0.1,
                   q_std=wl.STRESS_TEMPERATURE[alpha][ti] / math.sqrt(128))
    inp = dict(inp, workload=w)
    q = wl.fresh_query(w, inp, seed=5005 + 10 * ti + int(alpha * 100))
    inp["q"] = q
    print(f"[fullsize] stress alpha={alpha} T#{ti} {policy} k={top_k}", flush=True)
    gpu = run_gpu(inp, policy, top_k=w.top_k)
    check_properties(inp, gpu, policy, w.top_k)
    check_pair(inp, gpu, 0, 0, policy, top_k=w.top_k, check_meta=(ti == 0 and alpha == 1.25))
    check_pair(inp, gpu, 31, 7, policy, top_k=w.top_k, check_meta=False)
    if policy == "topk":
        decoder_matches(inp, gpu, policy, alpha, w.top_k, w.delta, w.scale, q)


@pytest.mark.parametrize("policy", ["topk", "dense", "gauss_mass"])
def test_million_token_row(policy):
    # one 1M-token row (65536 pages): the dense decode splits it into 4096
    # runs of 256 token slots, past the 2048 whose candidate offsets fit in LDS
    # at once; top-8192 takes the separate selection and decode
    w = wl.CONFIGS["long1m"]
    if policy == "dense":
        w = wl.variant(w, policy="dense")
    elif policy == "gauss_mass":
        w = wl.variant(w, policy="gauss_mass", alpha=2.0, delta=1e-4)
    print(f"[fullsize] long1m {policy}: generating", flush=True)
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, policy)
    check_properties(inp, gpu, policy, w.top_k)
    print(f"[fullsize] long1m {policy}: oracle pair b0 g0", flush=True)
    check_pair(inp, gpu, 0, 0, policy)
