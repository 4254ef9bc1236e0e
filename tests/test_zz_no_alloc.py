"""ekv_decode_step_noalloc (the decode step for callers that cannot allocate
device memory) against ekv_decode_step with a caller workspace: two calls in a
row on the library's per-device scratch, the second on a smaller input, each
bit-identical to the workspace entry point on the same inputs (both run the
same kernels)."""
import pytest
import torch

from sparse_kv_cache_page_amd import binding as B
from sparse_kv_cache_page_amd import workloads as wl
from sparse_kv_cache_page_amd.binding import CacheShape

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(batch, seq_len, top_k, seed):
    w = wl.variant("gqa", batch=batch, seq_len=seq_len, top_k=top_k, planted_per_kv_head=16,
                   name=f"noalloc_b{batch}_l{seq_len}", seed=seed)
    inp = wl.make_inputs(w, device=DEV)
    s = CacheShape(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                   inp["max_pages"], inp["num_phys_pages"], torch.bfloat16)
    return w, inp, s


def _buffers(s):
    Bt, Hq, Hkv, d, mp, Np = (s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim,
                              s.max_pages_per_seq, s.num_phys_pages)
    return {"kmin": torch.empty(Np, Hkv, d, dtype=s.kv_dtype, device=DEV),
            "kmax": torch.empty(Np, Hkv, d, dtype=s.kv_dtype, device=DEV),
            "ubg": torch.full((Bt, Hkv, mp), float("nan"), device=DEV),
            "sel": torch.full((Bt, Hkv, mp), -7, dtype=torch.int32, device=DEV),
            "n_sel": torch.full((Bt, Hkv), -7, dtype=torch.int32, device=DEV),
            "out": torch.full((Bt, Hq, d), float("nan"), device=DEV),
            "tau": torch.full((Bt, Hq), float("nan"), device=DEV),
            "n_support": torch.full((Bt, Hq), -7, dtype=torch.int32, device=DEV)}


def _run(w, inp, s, noalloc):
    o = _buffers(s)
    B.build_page_meta(s, inp["K"], inp["block_table"], inp["seq_lens"], o["kmin"], o["kmax"])
    args = (s, inp["q"], w.scale, w.alpha, inp["K"], inp["V"], inp["block_table"],
            inp["seq_lens"], w.top_k, o["kmin"], o["kmax"], o["ubg"], o["sel"], o["n_sel"],
            o["out"])
    if noalloc:
        B.decode_step_noalloc(*args, tau=o["tau"], n_support=o["n_support"])
    else:
        ws = torch.zeros(B.step_workspace_bytes(s, w.top_k), dtype=torch.uint8, device=DEV)
        B.decode_step(*args, ws, tau=o["tau"], n_support=o["n_support"])
    torch.cuda.synchronize()
    return o


def _same(a, b, s):
    assert torch.equal(a["n_sel"], b["n_sel"])
    for bb in range(s.batch):
        for g in range(s.num_kv_heads):
            n = int(a["n_sel"][bb, g])
            assert torch.equal(a["sel"][bb, g, :n], b["sel"][bb, g, :n]), (bb, g)
    assert torch.equal(a["out"], b["out"])
    assert torch.equal(a["tau"], b["tau"])
    assert torch.equal(a["n_support"], b["n_support"])
    assert bool(torch.isfinite(a["out"]).all())


def test_noalloc_step_matches_workspace_step_twice():
    # the first case is the larger one: the second call reuses scratch that the
    # first left full of its own bounds and candidates
    for batch, seq_len, top_k, seed in ((8, 20000, 96, 61), (3, 5000, 40, 62)):
        w, inp, s = _case(batch, seq_len, top_k, seed)
        need = B.step_workspace_bytes(s, top_k)
        assert need <= B.NOALLOC_SCRATCH_BYTES
        print(f"[noalloc] batch {batch} len {seq_len} top-{top_k}: {need} scratch bytes",
              flush=True)
        got = _run(w, inp, s, noalloc=True)
        ref = _run(w, inp, s, noalloc=False)
        _same(got, ref, s)
