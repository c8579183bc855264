"""The tree-size controller on measured times (BASTION, "Controllore Online
del Budget Consapevole dell'Hardware"): T_verify(N) is timed on the GPU for a
small cache, and the library's controller -- fed the surrogate curve of the
GPU best-first trees -- must pick the same N as the oracle's controller fed
the oracle's trees, on the same measured times.  The plan-following time
model is then calibrated on those times through the library and must match
the oracle's restatement of it."""

import time

import numpy as np
import pytest
import torch
from scipy.optimize import least_squares

from oracle import verify_oracle as vo

pytestmark = pytest.mark.gpu


def test_controller_picks_the_oracle_n_on_measured_times(gpu_lib):
    ops = gpu_lib
    B, Hq, Hkv, D, L, NMAX = 2, 16, 4, 128, 8192, 48
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    kc = torch.randn(B, Hkv, L, D, device=dev, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, L, D, device=dev, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(77)
    K, T = 10, 4
    prob = rng.dirichlet(np.full(T, 0.4), size=(B, K)).astype(np.float32)
    tok = rng.integers(0, 1000, (B, K, T)).astype(np.int32)
    prob_d, tok_d = torch.from_numpy(prob).to(dev), torch.from_numpy(tok).to(dev)
    print("case controller: trees", flush=True)
    parent_all, _, rho_all, _ = ops.build_draft_tree(prob_d, tok_d, NMAX)
    torch.cuda.synchronize()
    rho_gpu = rho_all.cpu().numpy()
    rho_ora = np.stack([vo.best_first_tree(prob[b], tok[b], NMAX)[2] for b in range(B)])
    np.testing.assert_array_equal(rho_gpu, rho_ora)
    a_gpu = np.cumsum(rho_gpu.astype(np.float64).mean(axis=0))
    a_ora = np.cumsum(rho_ora.astype(np.float64).mean(axis=0))

    times = []
    for N in range(1, NMAX + 1):
        parent = ops.build_draft_tree(prob_d, tok_d, N)[0]
        q = torch.randn(B, Hq, N, D, device=dev, generator=g).to(torch.bfloat16)
        kd = torch.randn(B, Hkv, N, D, device=dev, generator=g).to(torch.bfloat16)
        vd = torch.randn(B, Hkv, N, D, device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty_like(q)
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device=dev)
        desc = ops.make_desc(q, kc, vc, kd, vd, out)
        ws = torch.empty(ops.workspace_size(desc, L), dtype=torch.uint8, device=dev)
        for _ in range(3):
            ops.verify_attn_dense(q, kc, vc, kd, vd, parent, out=out, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            ops.verify_attn_dense(q, kc, vc, kd, vd, parent, out=out, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) / 10)
    print(f"case controller: measured T(1)={times[0] * 1e6:.1f} us .. T({NMAX})={times[-1] * 1e6:.1f} us", flush=True)
    t = np.array(times)
    for t_draft in (0.0, t[0], 4 * t[0]):
        n_lib = ops.choose_tree_size(a_gpu, t, t_draft=t_draft, l_ar=t[0])
        n_ora, _ = vo.choose_tree_size(a_ora.astype(np.float32), t, t_draft=t_draft, l_ar=t[0])
        assert n_lib == n_ora, (t_draft, n_lib, n_ora)

    # calibrate the plan-following model on the measured times through the
    # library, and check the library's estimate against the oracle's model
    desc1 = ops.make_desc(torch.empty(B, Hq, 1, D, dtype=torch.bfloat16, device=dev), kc, vc,
                          torch.empty(B, Hkv, 1, D, dtype=torch.bfloat16, device=dev),
                          torch.empty(B, Hkv, 1, D, dtype=torch.bfloat16, device=dev),
                          torch.empty(B, Hq, 1, D, dtype=torch.bfloat16, device=dev))
    ns = np.arange(1, NMAX + 1)

    def model(p):
        bw, cs, ct, c0 = np.exp(p)
        return np.array([ops.verify_time_model(desc1, L, bw, cs, ct, c0, int(n)) for n in ns])
    fit = least_squares(lambda p: np.log(model(p)) - np.log(t), x0=np.log([5e12, 1e15, 4e14, 5e-6]),
                        bounds=(np.log([1e11, 1e12, 1e12, 1e-8]), np.log([2e13, 5e15, 5e15, 1e-2])))
    bw, cs, ct, c0 = np.exp(fit.x)
    got = model(fit.x)
    want = np.array([vo.verify_time_plan(B, Hq, Hkv, D, L, int(n), 2, bw, cs, ct, c0) for n in ns])
    np.testing.assert_allclose(got, want, rtol=1e-12)
    print(f"case controller: fitted model max residual {np.max(np.abs(got / t - 1)):.3f}", flush=True)
