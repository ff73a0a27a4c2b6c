"""The inverse-coefficient experiment (learning kappa through the
differentiable solve) against its oracle, oracle.inverse (pinned by
tests/test_oracle_inverse_pins.py):
matrix values, loss and gradient at a fixed theta, the first Adam steps, and
recovery of kappa on a 32 x 32 grid."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import banner, relerr
from oracle.inverse import Reference, adam

pytestmark = pytest.mark.gpu


def _setup(N, B, beta=1e-6, seed=11):
    from differentiable_sparse_linear_amd import inverse as inv
    F = np.random.default_rng(seed).standard_normal((B, N * N))
    model = inv.DiffusionInverse(N, torch.from_numpy(F).cuda(), beta=beta)
    th_true = inv.true_log_kappa(N)
    model.observe(torch.from_numpy(th_true).cuda())
    ref = Reference(N, F, th_true, beta)
    return inv, model, ref, th_true


def test_inverse_values_loss_and_gradient(hip):
    banner("inverse: gradient")
    N, B = 16, 4
    inv, model, ref, th_true = _setup(N, B)
    theta = 0.3 * th_true + 0.1 * np.random.default_rng(3).standard_normal(N * N)
    v = model.values(torch.from_numpy(theta).cuda()).cpu().numpy()
    vw = W.varcoef_diffusion((N, N), np.exp(theta))[2][0]
    assert relerr(v, vw) <= 1e-14
    assert relerr(model.u_obs.cpu().numpy(), ref.u_obs) <= 1e-10
    t = torch.from_numpy(theta).cuda().requires_grad_(True)
    L = model.loss(t)
    L.backward()
    loss, g = ref.loss_grad(theta)
    assert abs(L.item() - loss) <= 1e-8 * loss
    assert relerr(t.grad.cpu().numpy(), g) <= 1e-7


def test_inverse_adam_steps_match_reference(hip):
    banner("inverse: Adam trajectory")
    N, B, steps = 16, 4, 15
    inv, model, ref, th_true = _setup(N, B)
    out = inv.recover(N=N, B=B, steps=steps, lr=0.05, beta=1e-6, history=True)
    thetas, losses = adam(ref, steps, 0.05)
    for k in range(steps):
        assert relerr(out["history"][k].cpu().numpy(), thetas[k]) <= 1e-6, k
        assert abs(out["loss"][k] - losses[k]) <= 1e-7 * losses[k], k


def test_inverse_recovers_kappa(hip):
    banner("inverse: recovery 32x32")
    from differentiable_sparse_linear_amd import inverse as inv
    out = inv.recover(N=32, B=8, steps=300, lr=0.05, beta=1e-6)
    banner(f"kappa error {out['kappa_rel_err_start']:.3f} -> {out['kappa_rel_err']:.4f} "
           f"in {out['wall_s']:.2f} s")
    assert out["kappa_rel_err"] < 0.01
    assert out["loss"][-1] < 1e-3 * out["loss"][0]
