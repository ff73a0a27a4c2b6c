"""Lanczos eigenpairs (sla_eigsh) and the eigenvalue gradient
(sla_eigsh_adjoint, Hellmann-Feynman on the pattern) against oracle.eigen and
the closed-form Laplacian spectrum; at 1e6 unknowns, the eigen-residual
recomputed by the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from dense_ref import laplacian_eigval_2d
from gpu_helpers import banner, relerr, to_dev
from oracle import eigen as E

pytestmark = pytest.mark.gpu


def _pattern(hip, rp, col):
    return hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda())


def test_eigsh_laplacian_closed_form(hip):
    banner("eigsh laplacian")
    N = 32
    rp, col, val = W.laplacian_2d(N)
    pat = _pattern(hip, rp, col)
    lam = np.sort([laplacian_eigval_2d(N, j, k) for j in range(1, N + 1)
                   for k in range(1, N + 1)])
    v = torch.from_numpy(val[0]).cuda()
    ev, X, info = pat.eigsh(v, k=1, tol=1e-10, ncv=80)
    assert info["return"] == hip.SLA_OK
    assert abs(ev[0, 0].item() - lam[0]) <= 1e-10 * lam[0]
    ev, X, info = pat.eigsh(v, k=1, largest=True, tol=1e-10, ncv=80)
    assert abs(ev[0, 0].item() - lam[-1]) <= 1e-10 * lam[-1]


@pytest.mark.parametrize("largest", [False, True])
def test_eigsh_and_gradient_match_oracle(hip, largest):
    banner(f"eigsh varcoef largest={largest}")
    rng = np.random.default_rng(51)
    rp, col, val = W.varcoef_diffusion((20, 20), np.exp(0.5 * rng.standard_normal(400)))
    pat = _pattern(hip, rp, col)
    w, V = E.eigsh(rp, col, val[0], k=3, largest=largest)
    v = torch.from_numpy(val[0].copy()).cuda().requires_grad_(True)
    ev, X, = hip.sparse_eigsh(pat, v, k=3, largest=largest, tol=1e-11, ncv=100)
    assert relerr(ev.detach().cpu().numpy()[0], w) <= 1e-10
    Xh = X.cpu().numpy()[0]
    for q in range(3):
        assert abs(abs(float(Xh[q] @ V[q])) - 1.0) <= 1e-8, q
    g = np.array([1.0, 0.5, -0.25])
    (ev[0] * torch.from_numpy(g).cuda()).sum().backward()
    got = v.grad.cpu().numpy()
    assert relerr(got, E.eig_grad(rp, col, Xh, g)) <= 1e-12  # same vectors
    assert relerr(got, E.eig_grad(rp, col, V, g)) <= 1e-7    # the oracle's vectors


def test_eigsh_large_residual(hip):
    """The largest eigenpair of the 1e6-DOF diffusion matrix: the oracle
    recomputes ||A v - lambda v|| / lambda and the Rayleigh quotient."""
    banner("eigsh 1e6")
    p = W.config(2)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"])
    ev, X, info = pat.eigsh(d["val"], k=1, largest=True, tol=1e-8, ncv=60, max_restarts=40)
    assert info["return"] == hip.SLA_OK
    lam = ev[0, 0].item()
    x = X.cpu().numpy()[0, 0]
    ax = O.spmv(p.row_ptr, p.col, p.values[0], x)
    assert abs(np.linalg.norm(x) - 1.0) <= 1e-12
    assert np.linalg.norm(ax - lam * x) <= 1e-7 * lam
    assert abs(O.dot(x, ax) - lam) <= 1e-12 * lam


def test_eigsh_arguments(hip):
    banner("eigsh arguments")
    rp, col, val = W.laplacian_2d(4)
    pat = _pattern(hip, rp, col)
    v = torch.from_numpy(val[0]).cuda()
    for kw in ({"k": 0}, {"k": 9}, {"k": 1, "ncv": 600}, {"k": 1, "tol": 0.0}):
        with pytest.raises(hip.SlaError):
            pat.eigsh(v, **kw)
    # single-vector Lanczos sees one copy of a repeated eigenvalue: on the
    # square Laplacian the smallest eight it returns are the distinct ones
    ev, X, info = pat.eigsh(v, k=8, ncv=16)
    w = np.unique(np.round(np.linalg.eigvalsh(E.dense(rp, col, val[0])), 12))
    assert relerr(ev.cpu().numpy()[0], w[:8]) <= 1e-12
    # distinct eigenvalues, basis = the whole space: exact after one cycle
    rng = np.random.default_rng(52)
    rp, col, val = W.varcoef_diffusion((4, 4), np.exp(rng.standard_normal(16)))
    pat = _pattern(hip, rp, col)
    ev, X, info = pat.eigsh(torch.from_numpy(val[0]).cuda(), k=8, ncv=16)
    w = np.sort(np.linalg.eigvalsh(E.dense(rp, col, val[0])))
    assert info["return"] == hip.SLA_OK and info["restarts"][0] == 0
    assert relerr(ev.cpu().numpy()[0], w[:8]) <= 1e-12


def test_eigsh_basis_kept_by_the_handle(hip):
    """The handle keeps the Lanczos basis: repeated calls reuse it (same
    workspace, bitwise the same pairs); a call with a larger basis grows it
    once, a smaller one after it does not shrink or reallocate it."""
    banner("eigsh basis reuse")
    N = 24
    rp, col, val = W.laplacian_2d(N)
    pat = _pattern(hip, rp, col)
    v = torch.from_numpy(val[0]).cuda()
    w0 = pat.workspace_bytes()
    ev1, X1, _ = pat.eigsh(v, k=2, tol=1e-10, ncv=40)
    w1 = pat.workspace_bytes()
    ev2, X2, _ = pat.eigsh(v, k=2, tol=1e-10, ncv=40)
    assert pat.workspace_bytes() == w1 > w0
    assert torch.equal(ev1, ev2) and torch.equal(X1, X2)
    ev3, _, _ = pat.eigsh(v, k=3, tol=1e-10, ncv=60)
    w3 = pat.workspace_bytes()
    assert w3 > w1
    ev4, X4, _ = pat.eigsh(v, k=2, tol=1e-10, ncv=40)
    assert pat.workspace_bytes() == w3
    assert torch.equal(ev4, ev1) and torch.equal(X4, X1)
    assert abs(ev3[0, 0].item() - ev1[0, 0].item()) <= 1e-10 * ev1[0, 0].item()
