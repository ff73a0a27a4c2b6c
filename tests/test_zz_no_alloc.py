"""The solve that allocates nothing (sla_solve_noalloc) against sla_solve.

The no-alloc entry point runs the same one-workgroup CG solver as sla_solve
on a handle, with its state in the library's fixed device scratch array
instead of the handle's workspace; x and the per-system results must be
those of sla_solve bit for bit.  Two calls in a row, the second smaller,
so the second reads an array that still holds the first call's contents;
then the same for fp32 with int64 row pointers, an initial guess, a zero
diagonal, an invalid pattern, and the size limits.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import banner, oracle_forward_adjoint, relerr, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _handle_solve(hip, p, d, **kw):
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p))
    x, info = pat.solve(d["val"], d["b"], tol=p.tol, maxit=p.maxit, method="cg",
                        precond=p.precond, check=False, **kw)
    torch.cuda.synchronize()
    pat.close()
    return x, info


def _noalloc_solve(hip, p, d, x0=None):
    x = torch.full_like(d["b"], float("nan")) if x0 is None else x0.clone()
    info = hip.solve_noalloc(d["rp"], d["col"], d["val"], d["b"], x, tol=p.tol, maxit=p.maxit,
                             precond=p.precond, use_x0=x0 is not None, check=False)
    torch.cuda.synchronize()
    return x, info


def _same(hip, p, x0=None):
    d = to_dev(p)
    kw = {} if x0 is None else {"x0": x0}
    xh, ih = _handle_solve(hip, p, d, **kw)
    xn, inn = _noalloc_solve(hip, p, d, x0=x0)
    assert torch.equal(xn, xh), p.name
    for key in ("iters", "spmv", "status"):
        assert np.array_equal(inn[key], ih[key]), (p.name, key)
    assert inn["return"] == ih["return"], p.name
    assert inn["form"] == "block"
    np.testing.assert_allclose(inn["relres"], ih["relres"], rtol=4e-16, atol=0)
    return xn, inn


def test_noalloc_equals_solve_two_calls(hip):
    """Config 3 (64 systems of 64 x 64, Jacobi-PCG) and then config 1 (one
    32 x 32 system, plain CG): smaller in n and in batch."""
    banner("no-alloc: config 3 (64 systems) then config 1")
    p3 = W.config(3, batch=64)
    x3, i3 = _same(hip, p3)
    assert np.all(i3["status"] == 0)
    r, _ = oracle_forward_adjoint(p3, systems=[5])
    assert relerr(x3.cpu().numpy()[5], r.x[0]) <= 1e-7
    p1 = W.config(1)
    x1, i1 = _same(hip, p1)
    r, _ = oracle_forward_adjoint(p1)
    assert i1["status"][0] == 0 and i1["iters"][0] == r.iters[0]
    assert relerr(x1.cpu().numpy()[0], r.x[0]) <= 1e-7


def test_noalloc_fp32_int64_and_initial_guess(hip):
    banner("no-alloc: fp32 with int64 row pointers, then an initial guess")
    p = W.config(3, batch=16).astype(np.float32)
    p = W.Problem(p.name, p.n, p.row_ptr.astype(np.int64), p.col, p.values, p.b, p.x_t,
                  method="cg", precond="jacobi", tol=1e-5, maxit=p.maxit)
    _same(hip, p)
    q = W.config(1)
    x0 = torch.from_numpy(np.random.default_rng(4).uniform(-1, 1, (1, q.n))).cuda()
    _same(hip, q, x0=x0)


def test_noalloc_status_paths(hip):
    banner("no-alloc: zero diagonal, invalid pattern, limits")
    p = W.config(1)
    v = p.values.copy()
    v[0, int(np.searchsorted(p.col[p.row_ptr[7]:p.row_ptr[8]], 7)) + int(p.row_ptr[7])] = 0.0
    z = W.Problem("zero_diag", p.n, p.row_ptr, p.col, v, p.b, p.x_t, method="cg",
                  precond="jacobi", tol=p.tol, maxit=p.maxit)
    _, info = _same(hip, z)
    assert info["return"] == hip.SLA_ERR_ZERO_DIAG
    d = to_dev(p)
    bad = d["col"].clone()
    bad[10], bad[11] = d["col"][11], d["col"][10]
    x = torch.zeros_like(d["b"])
    with pytest.raises(hip.SlaError) as ei:
        hip.solve_noalloc(d["rp"], bad, d["val"], d["b"], x)
    assert ei.value.status == hip.SLA_ERR_PATTERN
    big = W.laplacian_2d(65)
    rp = torch.from_numpy(big[0]).cuda()
    col = torch.from_numpy(big[1]).cuda()
    vb = torch.ones(big[1].size, dtype=torch.float64, device="cuda")
    b = torch.ones(65 * 65, dtype=torch.float64, device="cuda")
    with pytest.raises(hip.SlaError) as ei:
        hip.solve_noalloc(rp, col, vb, b, torch.zeros_like(b))
    assert ei.value.status == hip.SLA_ERR_TOO_LARGE
    # and a good call after the failures
    _same(hip, p)
