"""Pins of oracle.inverse (the inverse-coefficient experiment's checker):
checks against central differences, closed forms and a library routine --
never against the module itself.  Planted mistakes in copies of the module
must each be rejected by at least one pin.  CPU only.

  I1  the chain rule values -> kappa: for a fixed G, L(kappa) =
      sum_k G_k values_k(kappa) with the values assembled by the workload
      generator; grad_kappa(G) against central differences of L in kappa.
  I2  loss_grad against central differences of the loss in theta (4 x 4
      grid, two forcings, the smoothness term on), relative error <= 1e-6.
  I3  Adam's first step from theta = 0 in closed form: m_hat = g and
      v_hat = g^2, so theta_1 = -lr g / (|g| + eps) per component.
  I4  Adam on a separable quadratic against torch.optim.Adam (float64,
      CPU) over 25 steps.
  I5  at the true coefficient with no smoothness term the loss and the
      gradient vanish (to the solve tolerance).
"""
import importlib.util
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

SRC = os.path.join(os.path.dirname(oracle.__file__), "inverse.py")


def _module(text=None, name="oracle.inverse"):
    """oracle.inverse, or a copy of its source with a planted mistake."""
    if text is None:
        import oracle.inverse as inv
        return inv
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(text, SRC, "exec"), mod.__dict__)
    return mod


def _rel(a, b):
    a, b = np.ravel(a), np.ravel(b)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _eps(v):
    return 1e-6 * max(1.0, abs(float(v)))


def pin_i1_grad_kappa_fd(inv):
    rng = np.random.default_rng(41)
    for N in (4, 5):
        kap = np.exp(0.7 * rng.standard_normal(N * N))
        rp, col, vals = W.varcoef_diffusion((N, N), kap)
        G = rng.standard_normal(col.size)
        got = inv.grad_kappa(N, rp, col, kap, G)
        fd = np.zeros(N * N)
        for c in range(N * N):
            e = _eps(kap[c])
            kp, km = kap.copy(), kap.copy()
            kp[c] += e
            km[c] -= e
            Lp = G @ W.varcoef_diffusion((N, N), kp)[2][0]
            Lm = G @ W.varcoef_diffusion((N, N), km)[2][0]
            fd[c] = (Lp - Lm) / (2 * e)
        assert _rel(got, fd) <= 1e-7, f"I1 N={N}: {_rel(got, fd):.2e}"


def _small_reference(inv, beta):
    N = 4
    rng = np.random.default_rng(42)
    F = rng.standard_normal((2, N * N))
    th_true = 0.5 * rng.standard_normal(N * N)
    return inv.Reference(N, F, th_true, beta, tol=1e-14, maxit=1000), th_true, rng


def pin_i2_loss_grad_fd(inv):
    ref, th_true, rng = _small_reference(inv, beta=1e-2)
    theta = th_true + 0.4 * rng.standard_normal(th_true.size)
    _, g = ref.loss_grad(theta)
    fd = np.zeros_like(theta)
    for c in range(theta.size):
        e = _eps(theta[c])
        tp, tm = theta.copy(), theta.copy()
        tp[c] += e
        tm[c] -= e
        fd[c] = (ref.loss_grad(tp)[0] - ref.loss_grad(tm)[0]) / (2 * e)
    assert _rel(g, fd) <= 1e-6, f"I2: {_rel(g, fd):.2e}"


def pin_i3_adam_first_step(inv):
    ref, _, _ = _small_reference(inv, beta=1e-2)
    lr, eps = 0.05, 1e-8
    thetas, losses = inv.adam(ref, 1, lr, eps=eps)
    L0, g = ref.loss_grad(np.zeros(ref.N * ref.N))
    assert losses[0] == L0
    assert _rel(thetas[0], -lr * g / (np.abs(g) + eps)) <= 1e-15, "I3"


class _Quadratic:
    """L(theta) = 1/2 sum_i w_i (theta_i - c_i)^2 on 3 x 3 = 9 entries."""

    def __init__(self):
        rng = np.random.default_rng(43)
        self.N = 3
        self.w = rng.uniform(0.5, 4.0, 9)
        self.c = rng.standard_normal(9)

    def loss_grad(self, th):
        d = th - self.c
        return 0.5 * float(np.sum(self.w * d * d)), self.w * d


def pin_i4_adam_against_torch(inv):
    q = _Quadratic()
    lr, steps = 0.1, 25
    thetas, _ = inv.adam(q, steps, lr)
    t = torch.zeros(9, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([t], lr=lr, betas=(0.9, 0.999), eps=1e-8)
    w = torch.from_numpy(q.w)
    c = torch.from_numpy(q.c)
    for k in range(steps):
        opt.zero_grad()
        (0.5 * torch.sum(w * (t - c) ** 2)).backward()
        opt.step()
        assert _rel(thetas[k], t.detach().numpy()) <= 1e-12, f"I4 step {k}"


def pin_i5_zero_at_truth(inv):
    ref, th_true, _ = _small_reference(inv, beta=0.0)
    L, g = ref.loss_grad(th_true)
    assert L <= 1e-20, f"I5 loss {L:.2e}"
    _, g1 = ref.loss_grad(th_true + 0.1)
    assert np.linalg.norm(g) <= 1e-8 * max(np.linalg.norm(g1), 1e-300), "I5 gradient"


PINS = [pin_i1_grad_kappa_fd, pin_i2_loss_grad_fd, pin_i3_adam_first_step,
        pin_i4_adam_against_torch, pin_i5_zero_at_truth]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(_module())


MUTANTS = {
    "drop_wall_faces": ("        dk[c] += walls[c] * G[pos[(c, c)]]\n",
                        "        dk[c] += 0.0 * G[pos[(c, c)]]\n"),
    "harmonic_derivative_wrong_cell": ("dk[x] += dldf * 2.0 * kb * kb / (ka + kb) ** 2",
                                       "dk[x] += dldf * 2.0 * ka * ka / (ka + kb) ** 2"),
    "face_gradient_sign": ("- G[pos[(x, y)]] - G[pos[(y, x)]]",
                           "+ G[pos[(x, y)]] + G[pos[(y, x)]]"),
    "drop_log_chain": ("adj.grad_values.sum(axis=0)) * kap", "adj.grad_values.sum(axis=0))"),
    "drop_smoothness_gradient": ("        np.add.at(g, self.b, -self.beta * d)\n", ""),
    "misfit_not_scaled": ("gx = (r.x - self.u_obs) / self.scale", "gx = (r.x - self.u_obs)"),
    "adam_no_bias_correction": ("mh = m / (1 - b1 ** t)", "mh = m"),
    "adam_v_not_squared": ("v = b2 * v + (1 - b2) * g * g", "v = b2 * v + (1 - b2) * np.abs(g)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    mod = _module(src.replace(old, new), name=f"oracle.inverse_{name}")
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
