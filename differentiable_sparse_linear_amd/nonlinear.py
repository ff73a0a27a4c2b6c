"""Differentiable nonlinear solve F(u, theta) = 0.

The torch-sla pages (gist.science explainer, Methodology section 2,
nonlinear systems) give the backward pass of a nonlinear system as one
adjoint linear solve J^T lambda = dL/du plus one vector-Jacobian product,
independent of the number of nonlinear iterations.  Here:

* forward: Newton's method, J(u_k) delta = F(u_k), u_{k+1} = u_k - delta,
  from u_0 (zero by default) until ||F(u_k)|| <= tol ||F(u_0)||, each
  Jacobian solve by the library (CG + Jacobi for a symmetric Jacobian,
  BiCGStab otherwise), nothing recorded for autograd;
* backward: lambda from J(u)^T lambda = dL/du by the library (CG: J itself;
  BiCGStab: through the transpose map), then dL/dtheta = -lambda^T dF/dtheta,
  the vector-Jacobian product of the caller's residual at the solution (one
  evaluation of F with autograd).  Only u and theta are kept between the
  passes: memory O(n + nnz), whatever the Newton iteration count.

The caller supplies F (torch operations, differentiable in theta) and the
Jacobian's values on the pattern.  ``Semilinear`` is the model problem
F(u; v, c, f) = A(v) u + c * u^3 - f, whose product A(v) u goes through the
library's differentiable product.
"""
from __future__ import annotations

from typing import Callable, Sequence

import torch

from . import Pattern, SlaError, sparse_matvec


class NewtonSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, pattern: Pattern, residual: Callable, jac_values: Callable, opts: dict,
                u0, *params):
        tol, maxit = opts["tol"], opts["maxit"]
        lin = {"tol": opts["lin_tol"], "maxit": opts["lin_maxit"], "method": opts["method"],
               "precond": opts["precond"]}
        with torch.no_grad():
            u = torch.zeros(pattern.n, dtype=pattern.dtype, device=pattern.device) \
                if u0 is None else u0.detach().clone()
            F = residual(u, *params)
            norms = [float(torch.linalg.norm(F))]
            it = 0
            while norms[-1] > tol * norms[0] and it < maxit:
                J = jac_values(u, *params).contiguous()
                delta, info = pattern.solve(J, F.contiguous(), **lin)
                if int(info["status"][0]) < 0 or int(info["status"][0]) == 2:
                    raise SlaError(int(info["status"][0]), "Newton step")
                u = u - delta
                F = residual(u, *params)
                norms.append(float(torch.linalg.norm(F)))
                it += 1
        ctx.pattern, ctx.residual, ctx.jac_values, ctx.lin = pattern, residual, jac_values, lin
        ctx.newton_iters, ctx.norms = it, norms
        ctx.save_for_backward(u, *params)
        return u

    @staticmethod
    def backward(ctx, grad_u):
        u, *params = ctx.saved_tensors
        pattern, lin = ctx.pattern, ctx.lin
        with torch.no_grad():
            J = ctx.jac_values(u, *params).contiguous()
            if lin["method"] == "cg":
                lam, _ = pattern.solve(J, grad_u.contiguous(), **lin)
            else:
                _, lam, _ = pattern.solve_adjoint(J, u, grad_u.contiguous(), **lin)
        want = [i for i, p in enumerate(params) if ctx.needs_input_grad[5 + i]]
        grads = [None] * len(params)
        if want:
            with torch.enable_grad():
                ps = [p.detach().requires_grad_(i in want) for i, p in enumerate(params)]
                F = ctx.residual(u.detach(), *ps)
                got = torch.autograd.grad(F, [ps[i] for i in want], grad_outputs=-lam,
                                          allow_unused=True)
            for i, g in zip(want, got):
                grads[i] = g
        return (None, None, None, None, None, *grads)


def nonlinear_solve(pattern: Pattern, residual: Callable, jac_values: Callable,
                    params: Sequence[torch.Tensor], u0=None, tol: float = 1e-10, maxit: int = 50,
                    method: str = "cg", precond: str = "jacobi", lin_tol: float = 1e-12,
                    lin_maxit: int = 10000) -> torch.Tensor:
    """u with F(u, *params) = 0, differentiable in params."""
    opts = {"tol": tol, "maxit": maxit, "method": method, "precond": precond,
            "lin_tol": lin_tol, "lin_maxit": lin_maxit}
    return NewtonSolve.apply(pattern, residual, jac_values, opts, u0, *params)


class Semilinear:
    """F(u; v, c, f) = A(v) u + c * u^3 - f on a pattern (one system; A SPD
    and c >= 0 make the Jacobian A + diag(3 c u^2) SPD)."""

    def __init__(self, pattern: Pattern):
        self.pattern = pattern
        self.diagpos = pattern.export_pattern()[0].long()

    def residual(self, u, v, c, f):
        return sparse_matvec(self.pattern, v, u) + c * u ** 3 - f

    def jac_values(self, u, v, c, f):
        return v.index_add(0, self.diagpos, 3.0 * c * u * u)

    def solve(self, v, c, f, **opts) -> torch.Tensor:
        return nonlinear_solve(self.pattern, self.residual, self.jac_values, (v, c, f), **opts)
