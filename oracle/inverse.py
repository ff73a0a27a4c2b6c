"""Oracle of the inverse-coefficient experiment -- TEST INFRASTRUCTURE ONLY
(same rules as the rest of ``oracle/``: only tests, the smoke check and the
benchmark's CPU baseline may use it; it shares nothing with the HIP path or
with differentiable_sparse_linear_amd.inverse).

The torch-sla pages (gist.science explainer, Results) report recovering a
diffusion coefficient by gradient descent through the differentiable solve.
The synthetic experiment checked here: the cell-centred operator
-div(kappa grad u) on an N x N grid (the harmonic-face stencil of the
seeded workload generator, workloads.varcoef_diffusion), kappa = exp(theta)
per cell, B forcing fields f_r observed through u_r = A(kappa)^-1 f_r, and

    L(theta) = sum_r 1/2 |u_r - u_obs_r|^2 / sum_r 1/2 |u_obs_r|^2
               + beta/2 sum over interior faces (theta_a - theta_b)^2,

minimised by Adam from theta = 0.  The solves and adjoints are the oracle's
(oracle.solve, oracle.adjoint: the gradient on the pattern, Methodology
section 2); the chain rule from the values to kappa is written out below;
Adam follows Kingma & Ba (2015), Algorithm 1.

Chain rule.  An interior face between cells a and b has coefficient
f = 2 k_a k_b / (k_a + k_b); it enters A_ab = A_ba = -f and A_aa, A_bb with
+f, so dL/df = G_aa + G_bb - G_ab - G_ba (G = dL/dvalues on the pattern),
and df/dk_a = 2 k_b^2 / (k_a + k_b)^2.  A wall face of cell a has f = k_a
and enters A_aa only (once per wall the cell touches).  Finally
dL/dtheta = dL/dk * k.

Pinned by tests/test_oracle_inverse_pins.py (central differences of the
chain rule and of the loss, Adam's closed-form first step, Adam against
torch.optim.Adam, the loss at the true coefficient).
"""
from __future__ import annotations

import numpy as np

import workloads as W

from . import adjoint, solve


def interior_faces(N: int):
    """(a, b): the cells on either side of each interior face, x-faces
    first, cells numbered x fastest."""
    i = np.arange(N * N)
    ix, iy = i % N, i // N
    h = i[ix < N - 1]
    v = i[iy < N - 1]
    return np.concatenate([h, v]), np.concatenate([h + 1, v + N])


def grad_kappa(N: int, rp, col, kap, G):
    """dL/dkappa from G = dL/dvalues on the pattern (rp, col) of the N x N
    harmonic-face operator with cell coefficients kap."""
    n = N * N
    rows = np.repeat(np.arange(n), np.diff(rp))
    pos = {(int(r), int(c)): k for k, (r, c) in enumerate(zip(rows, col))}
    dk = np.zeros(n)
    a, b = interior_faces(N)
    for x, y in zip(a, b):
        ka, kb = kap[x], kap[y]
        dldf = G[pos[(x, x)]] + G[pos[(y, y)]] - G[pos[(x, y)]] - G[pos[(y, x)]]
        dk[x] += dldf * 2.0 * kb * kb / (ka + kb) ** 2
        dk[y] += dldf * 2.0 * ka * ka / (ka + kb) ** 2
    i = np.arange(n)
    ix, iy = i % N, i // N
    walls = (ix == 0).astype(int) + (ix == N - 1) + (iy == 0) + (iy == N - 1)
    for c in np.nonzero(walls)[0]:
        dk[c] += walls[c] * G[pos[(c, c)]]
    return dk


class Reference:
    """The experiment's loss and gradient on the CPU for forcing [B, N * N]
    and the true log-coefficient theta_true [N * N]."""

    def __init__(self, N, forcing, theta_true, beta, tol=1e-10, maxit=10000):
        self.N, self.F, self.beta, self.tol, self.maxit = N, forcing, beta, tol, maxit
        self.B = forcing.shape[0]
        rp, col, vt = W.varcoef_diffusion((N, N), np.exp(theta_true))
        self.rp, self.col = rp, col
        self.u_obs = solve(rp, col, np.repeat(vt, self.B, axis=0), forcing, "cg", "jacobi",
                           1e-12, maxit).x
        self.scale = 0.5 * np.sum(self.u_obs ** 2)
        self.a, self.b = interior_faces(N)

    def loss_grad(self, theta):
        """(L(theta), dL/dtheta)."""
        kap = np.exp(theta)
        _, _, vals = W.varcoef_diffusion((self.N, self.N), kap)
        V = np.repeat(vals, self.B, axis=0)
        r = solve(self.rp, self.col, V, self.F, "cg", "jacobi", self.tol, self.maxit)
        gx = (r.x - self.u_obs) / self.scale
        adj = adjoint(self.rp, self.col, V, r.x, gx, "cg", "jacobi", self.tol, self.maxit)
        g = grad_kappa(self.N, self.rp, self.col, kap, adj.grad_values.sum(axis=0)) * kap
        d = theta[self.a] - theta[self.b]
        np.add.at(g, self.a, self.beta * d)
        np.add.at(g, self.b, -self.beta * d)
        loss = 0.5 * np.sum((r.x - self.u_obs) ** 2) / self.scale + \
            0.5 * self.beta * np.sum(d * d)
        return loss, g


def adam(ref, steps, lr, b1=0.9, b2=0.999, eps=1e-8):
    """Kingma & Ba, Algorithm 1, from theta = 0 on ref.loss_grad (theta of
    ref.N * ref.N entries); returns (theta after each step, loss at each
    step's start)."""
    th = np.zeros(ref.N * ref.N)
    m = np.zeros_like(th)
    v = np.zeros_like(th)
    thetas, losses = [], []
    for t in range(1, steps + 1):
        loss, g = ref.loss_grad(th)
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh = m / (1 - b1 ** t)
        vh = v / (1 - b2 ** t)
        th = th - lr * mh / (np.sqrt(vh) + eps)
        thetas.append(th.copy())
        losses.append(loss)
    return thetas, losses
