"""Differentiable Newton solve of A(v) u + c u^3 = f (the nonlinear adjoint:
one J^T solve plus one vector-Jacobian product) against oracle.nonlinear:
the solution, the Newton iteration count and the gradients in v, c and f,
for a symmetric (CG) and a nonsymmetric (BiCGStab) operator."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import banner, relerr, to_dev
from oracle import nonlinear as NL

pytestmark = pytest.mark.gpu


def _case(hip, name):
    rng = np.random.default_rng(41)
    if name == "diffusion_32":
        rp, col, val = W.varcoef_diffusion((32, 32), np.exp(0.5 * rng.standard_normal(1024)))
        v, kw = val[0], dict(method="cg", precond="jacobi")
    else:
        p = W.config(4, size=32)
        rp, col, v = p.row_ptr, p.col, p.values[0] / 19.0
        kw = dict(method="bicgstab", precond="none")
    n = rp.shape[0] - 1
    c = rng.uniform(0.5, 2.0, n)
    f = 3.0 * rng.standard_normal(n)
    ut = rng.standard_normal(n)
    return rp, col, v, c, f, ut, kw


@pytest.mark.parametrize("name", ["diffusion_32", "convdiff_32"])
def test_nonlinear_solve_and_adjoint_match_oracle(hip, name):
    banner(f"nonlinear {name}")
    from differentiable_sparse_linear_amd.nonlinear import Semilinear
    rp, col, v, c, f, ut, kw = _case(hip, name)
    pat = hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda(),
                      build_transpose=True)
    model = Semilinear(pat)
    tv, tc, tf = (torch.from_numpy(a.copy()).cuda().requires_grad_(True) for a in (v, c, f))
    u = model.solve(tv, tc, tf, tol=1e-12, lin_tol=1e-13, **kw)
    loss = 0.5 * torch.sum((u - torch.from_numpy(ut).cuda()) ** 2)
    loss.backward()
    uo, it, norms = NL.newton(rp, col, v, c, f, tol=1e-12, lin_tol=1e-13, **kw)
    gv, gc, gf = NL.adjoint(rp, col, v, c, uo, uo - ut, lin_tol=1e-13, **kw)
    assert it >= 3
    assert u.grad_fn is not None
    assert relerr(u.detach().cpu().numpy(), uo) <= 1e-9
    assert relerr(tv.grad.cpu().numpy(), gv) <= 1e-7
    assert relerr(tc.grad.cpu().numpy(), gc) <= 1e-7
    assert relerr(tf.grad.cpu().numpy(), gf) <= 1e-7


def test_nonlinear_backward_keeps_only_the_solution(hip):
    """The backward pass needs u and the parameters only: the autograd graph
    of the Newton solve is one node whatever the Newton iteration count."""
    banner("nonlinear graph size")
    from differentiable_sparse_linear_amd.nonlinear import Semilinear
    rp, col, v, c, f, ut, kw = _case(hip, "diffusion_32")
    pat = hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda())
    model = Semilinear(pat)
    tv = torch.from_numpy(v.copy()).cuda().requires_grad_(True)
    tc = torch.from_numpy(c.copy()).cuda()
    for scale in (0.1, 3.0):  # fewer and more Newton iterations
        tf = torch.from_numpy(scale * f).cuda()
        u = model.solve(tv, tc, tf, **kw)
        node = u.grad_fn
        assert type(node).__name__ == "NewtonSolveBackward"
        assert len(node.saved_tensors) == 4  # u, v, c, f
