"""GPU parity of the Gaussian selection rules at non-integer gamma.

EntmaxKV summary page, §2.B (Gaussian-aware entmax selection): tau-hat solves
sum_p n_p E[(X_p - tau)_+^gamma] = 1.  For 1 < alpha < 2 with 1/(alpha-1) not
an integer the device evaluates E[(X - tau)_+^gamma] from a per-launch
Chebyshev table of I_f and I_{f+1} (f the fractional part of gamma) built by
quadrature, and the oracle by adaptive quadrature of the defining integral;
tau-hat, the selections (also stage-wise, from the GPU's own moments) and the
decode are compared with check_pair, at alpha = 1.7 (gamma = 1/0.7) and 1.4
(gamma = 2.5).  The oracle's quadrature costs ~0.2 ms per page and head, so
the rows are short; a row above the LDS staging limit (4096 pages) is checked
through the normalisation F(tau-hat) = 1 itself.
"""
import numpy as np
import pytest
import torch

from oracle import select
from sparse_kv_cache_page_amd import workloads as wl

from gpu_util import check_pair, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(seed, **kw):
    base = dict(name="small", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=128,
                page_size=16, lens_range=(100, 800), kv_dtype="bf16",
                q_std=2.0 / np.sqrt(128), scale=1.0, alpha=1.7, policy="gauss",
                clusters=16, planted_per_kv_head=0, permute_pool=True, seed=seed)
    base.update(kw)
    return wl.Workload(**base)


@pytest.mark.parametrize("alpha", [1.7, 1.4])
@pytest.mark.parametrize("policy,delta", [("gauss", 0.1), ("gauss_est", 0.1),
                                          ("gauss_mass", 1e-4)])
def test_gauss_fractional_gamma(policy, delta, alpha):
    w = small(811 + int(alpha * 10), alpha=alpha, policy=policy, delta=delta)
    inp = wl.make_inputs(w, device=DEV)
    print(f"[gauss_frac] {policy} alpha={alpha}", flush=True)
    gpu = run_gpu(inp, policy)
    for b in range(w.batch):
        check_pair(inp, gpu, b, 0, policy)


@pytest.mark.parametrize("alpha,page_size", [(1.7, 8), (1.4, 32), (1.2, 16)])
def test_gauss_fractional_gamma_page_sizes(alpha, page_size):
    # alpha = 1.2: gamma = 5, an integer above the unrolled ones (the run-time
    # recurrence from Phi and phi)
    w = small(823, alpha=alpha, policy="gauss_mass", delta=1e-3, page_size=page_size,
              lens_range=(60, 500))
    inp = wl.make_inputs(w, device=DEV)
    gpu = run_gpu(inp, "gauss_mass")
    for b in range(w.batch):
        check_pair(inp, gpu, b, 0, "gauss_mass")


def test_gauss_fractional_gamma_long_row():
    # 4500 pages: tau-hat read from global memory (no LDS staging); checked by
    # the oracle's F at the GPU's tau-hat and its sign change around it
    w = small(829, alpha=1.7, policy="gauss", delta=0.1, batch=1, lens_range=None)
    inp = wl.make_inputs(w, device=DEV, lens=[72000])
    gpu = run_gpu(inp, "gauss")
    a1 = float(np.float32(1.7)) - 1.0
    g = select.selection_gamma(float(np.float32(1.7)))
    n = (72000 + 15) // 16
    counts = np.full(n, 16.0)
    counts[-1] = 72000 - 16 * (n - 1)
    for h in (0, 3):
        th = float(gpu["tau_hat"][0, h])
        m = gpu["gm"][0, h, :n].cpu().numpy()
        v = gpu["gv"][0, h, :n].cpu().numpy()
        mu_z, sig_z = a1 * m, a1 * np.sqrt(v)
        F = select.gauss_F(th, mu_z, sig_z, counts, g)
        assert abs(F - 1.0) < 1e-10, (h, F)
        step = 1e-8 * max(1.0, abs(th))
        assert select.gauss_F(th - step, mu_z, sig_z, counts, g) > 1.0
        assert select.gauss_F(th + step, mu_z, sig_z, counts, g) < 1.0
