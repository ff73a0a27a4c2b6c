"""Oracle for the nonlinear adjoint -- TEST INFRASTRUCTURE ONLY (same rules
as the rest of ``oracle/``: only tests, the smoke check and the benchmark's
CPU baseline may use it; it shares nothing with the HIP path).

The torch-sla pages (gist.science explainer, Methodology section 2,
nonlinear systems) state that for F(u, theta) = 0 the backward pass is one
adjoint linear solve J^T lambda = dL/du plus one vector-Jacobian product,
whatever the number of nonlinear iterations.  The model problem here is the
semilinear system

    F(u; v, c, f) = A(v) u + c * u^3 - f = 0

(A on a CSR pattern with values v, c >= 0 per unknown, f the forcing),
whose Jacobian J = A(v) + diag(3 c u^2) is SPD when A is.

Forward: Newton's method from u_0 = 0: J(u_k) delta = F(u_k),
u_{k+1} = u_k - delta, until ||F(u_k)|| <= tol ||F(u_0)|| (= tol ||f||);
each linear solve by the oracle's Jacobi-PCG.
Backward, by the implicit-function theorem (dF/du du + dF/dtheta dtheta = 0):
solve J^T lambda = dL/du (J is symmetric, so by CG with J itself); then
dL/dtheta = -lambda^T dF/dtheta with dF/dv_k = u_j e_i for stored entry
k = (i, j), dF/dc = diag(u^3), dF/df = -I:
    dL/dv_k = -lambda_i u_j,   dL/dc = -lambda u^3,   dL/df = lambda.
"""
from __future__ import annotations

import numpy as np

from . import adjoint as linear_adjoint
from . import check_pattern, dot, grad_on_pattern, solve, spmv


def residual(row_ptr, col, v, c, f, u):
    return spmv(row_ptr, col, v, u) + c * u ** 3 - f


def jacobian_values(row_ptr, col, v, c, u):
    """Values of J = A(v) + diag(3 c u^2) on the same pattern."""
    n = np.asarray(row_ptr).shape[0] - 1
    st, diagpos = check_pattern(n, row_ptr, col)
    assert st == 0, "pattern without a diagonal"
    jv = np.array(v, dtype=np.float64, copy=True)
    jv[diagpos] += 3.0 * c * u * u
    return jv


def newton(row_ptr, col, v, c, f, tol=1e-10, maxit=50, lin_tol=1e-12, lin_maxit=10000,
           method="cg", precond="jacobi"):
    """Returns (u, newton iterations, residual norms ||F(u_k)||).  The
    Jacobian solves use `method` (CG for symmetric, BiCGStab otherwise)."""
    n = np.asarray(row_ptr).shape[0] - 1
    u = np.zeros(n)
    F = residual(row_ptr, col, v, c, f, u)
    norms = [np.sqrt(dot(F, F))]
    it = 0
    while norms[-1] > tol * norms[0] and it < maxit:
        J = jacobian_values(row_ptr, col, v, c, u)
        r = solve(row_ptr, col, J, F, method, precond, lin_tol, lin_maxit)
        u = u - r.x[0]
        F = residual(row_ptr, col, v, c, f, u)
        norms.append(np.sqrt(dot(F, F)))
        it += 1
    return u, it, norms


def adjoint(row_ptr, col, v, c, u, grad_u, lin_tol=1e-12, lin_maxit=10000, method="cg",
            precond="jacobi"):
    """(dL/dv [nnz], dL/dc [n], dL/df [n]) for dL/du = grad_u at the solution
    u.  lambda solves J^T lambda = grad_u: with CG J itself (symmetric), with
    BiCGStab the oracle's transposed system."""
    J = jacobian_values(row_ptr, col, v, c, u)
    if method == "cg":
        lam = solve(row_ptr, col, J, grad_u, method, precond, lin_tol, lin_maxit).x[0]
    else:
        lam = linear_adjoint(row_ptr, col, J, u, grad_u, method, precond, lin_tol,
                             lin_maxit).grad_b[0]
    grad_v = grad_on_pattern(row_ptr, col, lam, u)[0]  # -lambda_i u_j
    grad_c = -lam * u ** 3
    return grad_v, grad_c, lam
