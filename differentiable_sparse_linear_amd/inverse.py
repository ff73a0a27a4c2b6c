"""Inverse-coefficient learning through the differentiable solve.

The torch-sla pages (gist.science explainer, Results) report recovering a
diffusion coefficient by gradient descent through the solver.  This module
is that experiment on a synthetic problem: the cell-centred operator
-div(kappa grad u) on an N x N grid (harmonic-mean faces, Dirichlet walls
whose face coefficient is the cell's kappa, diagonal = sum of the four face
coefficients, unscaled), kappa = exp(theta) per cell, B forcing fields f_r
observed through u_r = A(kappa)^-1 f_r.  The loss

    L(theta) = sum_r 1/2 |u_r - u_obs_r|^2 / sum_r 1/2 |u_obs_r|^2
               + beta/2 sum over interior faces (theta_a - theta_b)^2

is minimised with Adam.  Every solve and its adjoint (the gradient on the
pattern, Methodology section 2) runs in the library's kernels through
``sparse_solve``; the assembly kappa -> matrix values is a few elementwise
tensor operations whose gradient torch's autograd forms.
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import Pattern, sparse_solve


def stencil_pattern(N: int):
    """CSR pattern of the five-point grid operator (columns ascending: south,
    west, centre, east, north) and the [n, 5] mask of stored slots."""
    n = N * N
    i = np.arange(n)
    ix, iy = i % N, i // N
    mask = np.stack([iy > 0, ix > 0, np.ones(n, bool), ix < N - 1, iy < N - 1], axis=1)
    offs = np.array([-N, -1, 0, 1, N])
    cols = (i[:, None] + offs[None, :])[mask].astype(np.int32)
    row_ptr = np.zeros(n + 1, dtype=np.int32)
    np.cumsum(mask.sum(axis=1), out=row_ptr[1:])
    return row_ptr, cols, mask


def true_log_kappa(N: int) -> np.ndarray:
    """A smooth log-coefficient on the cell centres (x fastest)."""
    c = (np.arange(N) + 0.5) / N
    X, Y = np.meshgrid(c, c)
    return (0.6 * np.sin(2 * np.pi * X) * np.sin(np.pi * Y)
            + 0.4 * np.cos(np.pi * X) * Y).reshape(-1)


def assemble_values(theta: torch.Tensor, N: int, mask: torch.Tensor) -> torch.Tensor:
    """Values [nnz] of the grid operator in the CSR order of stencil_pattern
    for kappa = exp(theta) (theta [N * N], x fastest)."""
    k = torch.exp(theta).reshape(N, N)  # [y, x]
    harm = lambda a, b: (2.0 * a * b) / (a + b)
    fx = harm(k[:, :-1], k[:, 1:])      # faces between x and x + 1
    fy = harm(k[:-1, :], k[1:, :])      # faces between y and y + 1
    west = torch.cat([k[:, :1], fx], dim=1)
    east = torch.cat([fx, k[:, -1:]], dim=1)
    south = torch.cat([k[:1, :], fy], dim=0)
    north = torch.cat([fy, k[-1:, :]], dim=0)
    diag = ((south + west) + east) + north
    slots = torch.stack([-south, -west, diag, -east, -north], dim=-1).reshape(N * N, 5)
    return slots[mask]


class DiffusionInverse:
    """The forward model and loss of the experiment on one device."""

    def __init__(self, N: int, forcing: torch.Tensor, beta: float = 1e-6, tol: float = 1e-10,
                 maxit: int = 10000):
        self.N, self.n = N, N * N
        self.B = forcing.shape[0]
        self.device = forcing.device
        rp, col, mask = stencil_pattern(N)
        self.nnz = int(col.shape[0])
        self.mask = torch.from_numpy(mask).to(self.device)
        self.pattern = Pattern(torch.from_numpy(rp).to(self.device),
                               torch.from_numpy(col).to(self.device), batch=self.B,
                               dtype=torch.float64)
        self.forcing = forcing.contiguous()
        self.beta, self.tol, self.maxit = beta, tol, maxit
        self.u_obs = None

    def values(self, theta: torch.Tensor) -> torch.Tensor:
        """Matrix values [nnz] in CSR order from theta = log kappa [n]."""
        return assemble_values(theta, self.N, self.mask)

    def solve(self, theta: torch.Tensor) -> torch.Tensor:
        v = self.values(theta)
        vb = v.unsqueeze(0).expand(self.B, self.nnz).reshape(-1)
        u = sparse_solve(self.pattern, vb, self.forcing.reshape(-1), tol=self.tol,
                         maxit=self.maxit, method="cg", precond="jacobi")
        return u.reshape(self.B, self.n)

    def observe(self, theta_true: torch.Tensor, tol: float = 1e-12):
        with torch.no_grad():
            v = self.values(theta_true)
            vb = v.unsqueeze(0).expand(self.B, self.nnz).contiguous()
            self.u_obs, info = self.pattern.solve(vb.reshape(-1), self.forcing.reshape(-1),
                                                  tol=tol, maxit=self.maxit, method="cg",
                                                  precond="jacobi")
            self.u_obs = self.u_obs.reshape(self.B, self.n)
        self.scale = 0.5 * float(torch.sum(self.u_obs * self.u_obs))

    def loss(self, theta: torch.Tensor) -> torch.Tensor:
        u = self.solve(theta)
        misfit = 0.5 * torch.sum((u - self.u_obs) ** 2) / self.scale
        t = theta.reshape(self.N, self.N)
        dx = t[:, :-1] - t[:, 1:]
        dy = t[:-1, :] - t[1:, :]
        return misfit + 0.5 * self.beta * (torch.sum(dx * dx) + torch.sum(dy * dy))


def recover(N: int = 64, B: int = 8, steps: int = 400, lr: float = 0.05, beta: float = 1e-6,
            seed: int = 11, device: str = "cuda:0", history: bool = False):
    """Run the experiment from kappa = 1; returns a dict with the relative L2
    error of kappa, the loss, the wall time and (optionally) theta after
    every step."""
    rng = np.random.default_rng(seed)
    forcing = torch.from_numpy(rng.standard_normal((B, N * N))).to(device)
    model = DiffusionInverse(N, forcing, beta=beta)
    theta_true = torch.from_numpy(true_log_kappa(N)).to(device)
    model.observe(theta_true)
    theta = torch.zeros(N * N, dtype=torch.float64, device=device, requires_grad=True)
    opt = torch.optim.Adam([theta], lr=lr)
    kt = torch.exp(theta_true)
    err0 = float(torch.linalg.norm(torch.exp(theta.detach()) - kt) / torch.linalg.norm(kt))
    hist, losses = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        opt.zero_grad()
        L = model.loss(theta)
        L.backward()
        opt.step()
        losses.append(L.detach())
        if history:
            hist.append(theta.detach().clone())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k = torch.exp(theta.detach())
    err = float(torch.linalg.norm(k - kt) / torch.linalg.norm(kt))
    out = {"N": N, "B": B, "steps": steps, "kappa_rel_err": err, "kappa_rel_err_start": err0,
           "loss": [float(l) for l in losses], "wall_s": wall, "theta": theta.detach()}
    if history:
        out["history"] = hist
    return out
