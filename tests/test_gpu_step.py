"""GPU tests of the fused decode step (ekv_decode_step).

The fused path must give bit-identical bounds and selections to the sequence
of separate entry points on the same inputs (same scoring arithmetic), and
the same outputs and thresholds (same decode kernels); it must leave its
workspace reusable (arrival counters back at zero) and replay correctly from
a captured HIP graph.  Selected pairs are also checked against the CPU oracle.
"""
import numpy as np
import pytest
import torch

from sparse_kv_cache_page_amd import binding as B
from sparse_kv_cache_page_amd import workloads as wl
from sparse_kv_cache_page_amd.engine import PagedEntmaxDecoder

from gpu_util import cache_shape, check_pair

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(seed, **kw):
    base = dict(name="small", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                page_size=16, lens_range=(37, 1500), kv_dtype="bf16",
                q_std=2.0 / np.sqrt(128), scale=1.0, alpha=1.5, policy="topk", top_k=9,
                planted_per_kv_head=8, permute_pool=True, seed=seed)
    base.update(kw)
    return wl.Workload(**base)


def separate_and_fused(inp, refresh):
    w = inp["workload"]
    s = cache_shape(inp)
    a = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale)
    f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, scale=w.scale,
                           fused=True)
    lens = inp["seq_lens"]
    if refresh:
        # metadata built for a shorter cache, then one token appended per row
        short = (lens - 1).clamp(min=1)
        a.build_meta(inp["K"], inp["block_table"], short)
        f.build_meta(inp["K"], inp["block_table"], short)
        last = ((lens + w.page_size - 1) // w.page_size - 1).to(torch.int32)
        a.build_meta(inp["K"], inp["block_table"], lens, first_page=last, span=1)
    else:
        a.build_meta(inp["K"], inp["block_table"], lens)
        f.build_meta(inp["K"], inp["block_table"], lens)
    a.step(inp["q"], inp["K"], inp["V"], inp["block_table"], lens)
    f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], lens, refresh_last_page=refresh)
    torch.cuda.synchronize()
    return a, f


def assert_same(a, f, inp):
    w = inp["workload"]
    assert torch.equal(a.n_sel, f.n_sel)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            n = int(a.n_sel[b, g])
            assert torch.equal(a.sel[b, g, :n], f.sel[b, g, :n])
            m = inp["npages"][b]
            assert torch.equal(a.ubg[b, g, :m], f.ubg[b, g, :m])
    assert torch.equal(a.out, f.out)
    assert torch.equal(a.tau, f.tau)
    assert torch.equal(a.n_support, f.n_support)
    assert torch.equal(a.kmin, f.kmin) and torch.equal(a.kmax, f.kmax)


@pytest.mark.parametrize("refresh", [False, True])
@pytest.mark.parametrize("kw", [
    dict(), dict(num_q_heads=16, num_kv_heads=2), dict(num_q_heads=4, num_kv_heads=4),
    dict(kv_dtype="f32", head_dim=64, q_std=2.0 / 8.0), dict(page_size=32, top_k=5),
    dict(page_size=1, lens_range=(3, 300), top_k=40), dict(top_k=1000),
    dict(page_size=1, lens_range=(3000, 6000), top_k=500, head_dim=64, q_std=0.25),
])
def test_fused_step_matches_separate(kw, refresh):
    w = small(201 + len(kw), **kw)
    inp = wl.make_inputs(w, device=DEV)
    a, f = separate_and_fused(inp, refresh)
    assert_same(a, f, inp)
    # and against the oracle on one pair
    gpu = dict(kmin=f.kmin, kmax=f.kmax, ub=None, ubg=f.ubg, sel=f.sel, n_sel=f.n_sel,
               out=f.out, tau=f.tau)
    b, g = w.batch - 1, w.num_kv_heads - 1
    _check_no_ub(inp, gpu, b, g)


def _check_no_ub(inp, gpu, b, g):
    from oracle import pipeline
    from gpu_util import OUT_TOL, TAU_TOL, TAU_TOL_REL, ulp_dist
    w = inp["workload"]
    G = w.group
    ref = pipeline.run_pair(inp, b, g, "topk")
    n = len(ref["phys"])
    assert ulp_dist(gpu["ubg"][b, g, :n].cpu().numpy(), ref["U"]).max() <= 1
    ns = int(gpu["n_sel"][b, g])
    assert gpu["sel"][b, g, :ns].cpu().tolist() == list(ref["sel"])
    tau = gpu["tau"][b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
    tol = np.maximum(TAU_TOL, TAU_TOL_REL * np.abs(ref["tau"]))
    assert np.all(np.abs(tau - ref["tau"]) <= tol)
    out = gpu["out"][b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
    for h in range(G):
        err = np.linalg.norm(out[h] - ref["o"][h]) / np.linalg.norm(ref["o"][h])
        assert err <= OUT_TOL


def test_fused_step_workspace_reusable():
    w = small(301, lens_range=(500, 2500))
    inp = wl.make_inputs(w, device=DEV)
    s = cache_shape(inp)
    f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, fused=True)
    f.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
    outs = []
    for i in range(3):
        f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
        torch.cuda.synchronize()
        outs.append((f.out.clone(), f.sel.clone(), f.n_sel.clone()))
        ncnt = s.batch * s.num_kv_heads
        assert int(f.step_ws[: 4 * ncnt].view(torch.int32).abs().sum()) == 0
        assert int(f.sel_ws[: 4 * ncnt].view(torch.int32).abs().sum()) == 0
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[2], outs[0][2])


def test_fused_step_graph_replay():
    # capture one fused step per layer; replay several times with eager work
    # in between; every replay must equal the eager result
    layers = []
    for i in range(2):
        w = small(401 + i, lens_range=(300, 2000))
        inp = wl.make_inputs(w, device=DEV)
        s = cache_shape(inp)
        f = PagedEntmaxDecoder(s, policy="topk", top_k=w.top_k, alpha=w.alpha, fused=True)
        f.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
        f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
        torch.cuda.synchronize()
        layers.append((inp, f, f.out.clone(), f.tau.clone()))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(stream):
        for inp, f, _, _ in layers:
            f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for inp, f, _, _ in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f.fused_step(inp["q"], inp["K"], inp["V"], inp["block_table"], inp["seq_lens"])
        graphs.append(g)
    for r in range(4):
        for (inp, f, out0, tau0), g in zip(layers, graphs):
            f.out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(f.out, out0) and torch.equal(f.tau, tau0), f"replay {r}"
            # unrelated eager work between replays
            torch.randn(1000, device=DEV).sum().item()


@pytest.mark.parametrize("alpha,q_std,L,policy", [
    (1.5, 0.001, 8192, "dense"),      # every token within 1 of the max: > 512 candidates
    (2.0, 0.002, 3000, "dense"),
    (1.25, 0.05, 20000, "dense"),
    (1.5, 0.18, 5000, "dense"),
    (1.5, 0.01, 30000, "topk"),
])
def test_fused_decode_against_oracle(alpha, q_std, L, policy):
    # ekv_entmax_decode_fused (tau / PV in the last workgroup of each pair)
    w = small(501, batch=2, num_q_heads=8, num_kv_heads=2, lens_range=None, seq_len=L,
              alpha=alpha, q_std=q_std, planted_per_kv_head=0, policy=policy, top_k=300)
    inp = wl.make_inputs(w, device=DEV)
    s = cache_shape(inp)
    dec = PagedEntmaxDecoder(s, policy=policy, top_k=w.top_k, alpha=alpha, scale=w.scale)
    dec.build_meta(inp["K"], inp["block_table"], inp["seq_lens"])
    if policy == "topk":
        dec.score(inp["q"], inp["block_table"], inp["seq_lens"])
        dec.select(inp["seq_lens"])
    ws = torch.zeros(B.decode_fused_workspace_bytes(s, dec.max_sel), dtype=torch.uint8,
                     device=DEV)
    out = torch.full_like(dec.out, float("nan"))
    tau = torch.full_like(dec.tau, float("nan"))
    dense = policy == "dense"
    for _ in range(2):   # the second call reuses the workspace as left by the first
        B.entmax_decode(s, inp["q"], w.scale, alpha, inp["K"], inp["V"], inp["block_table"],
                        inp["seq_lens"], out, ws, sel=None if dense else dec.sel,
                        n_sel=None if dense else dec.n_sel, max_sel=dec.max_sel, tau=tau,
                        fused=True)
        torch.cuda.synchronize()
    gpu = dict(kmin=dec.kmin, kmax=dec.kmax, ubg=dec.ubg, sel=dec.sel, n_sel=dec.n_sel, out=out,
               tau=tau)
    from oracle import pipeline
    from gpu_util import OUT_TOL, TAU_TOL, TAU_TOL_REL
    G = w.group
    for b, g in [(0, 0), (1, 1)]:
        ref = pipeline.run_pair(inp, b, g, policy)
        t = tau[b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
        tol = np.maximum(TAU_TOL, TAU_TOL_REL * np.abs(ref["tau"]))
        assert np.all(np.abs(t - ref["tau"]) <= tol), (t, ref["tau"])
        o = out[b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
        for h in range(G):
            err = np.linalg.norm(o[h] - ref["o"][h]) / np.linalg.norm(ref["o"][h])
            assert err <= OUT_TOL, err
