"""Pins for the oracle: checks against closed forms, dense solves, finite
differences and textbook bounds -- never against the oracle itself.

Each ``pin_*`` function raises AssertionError on a violation; the pytest
wrappers at the bottom run them, and ``test_oracle_mutants.py`` re-runs them
against deliberately broken oracle builds to show each plausible mistake is
caught.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from dense_ref import (laplacian_eigval_2d, laplacian_eigvec_2d, pattern_rows,
                       to_dense)


def _relerr(a, b):
    return float(np.linalg.norm(np.ravel(a) - np.ravel(b)) / max(np.linalg.norm(np.ravel(b)), 1e-300))


# --------------------------------------------------------------------------
# P1 -- SpMV against the closed-form Dirichlet Laplacian spectra (1D and 2D)
# --------------------------------------------------------------------------
def pin_p1_spmv_eigvecs():
    N = 16
    rp, col, val = W.varcoef_diffusion((N,), np.ones(N))
    h = np.pi / (N + 1)
    p = np.arange(1, N + 1)
    for j in (1, 5, 16):
        v = np.sin(j * p * h)
        lam = 2.0 - 2.0 * np.cos(j * h)
        y = O.spmv(rp, col, val, v)
        assert np.max(np.abs(y - lam * v)) <= 1e-14 * np.max(np.abs(v)) * 4, "1D eigenpair"
    N = 32
    rp, col, val = W.laplacian_2d(N)
    for (j, k) in [(1, 1), (3, 7), (32, 1), (17, 29)]:
        v = laplacian_eigvec_2d(N, j, k)
        lam = laplacian_eigval_2d(N, j, k)
        y = O.spmv(rp, col, val, v)
        assert np.max(np.abs(y - lam * v)) <= 1e-14 * 8, f"2D eigenpair {(j, k)}"


# --------------------------------------------------------------------------
# P2 -- SpMV against a dense product on random tiny CSR matrices
# --------------------------------------------------------------------------
def pin_p2_spmv_dense():
    rng = np.random.default_rng(11)
    for seed, n in [(1, 7), (2, 33), (3, 64)]:
        rp, col, val = W.random_csr(n, 0.2, seed, symmetric=False)
        A = to_dense(rp, col, val)
        x = rng.standard_normal(n)
        y = O.spmv(rp, col, val, x)
        ref = A @ x
        scale = np.abs(A) @ np.abs(x)
        assert np.all(np.abs(y - ref) <= 4e-16 * 8 * scale + 1e-300), "dense matvec"


def pin_p2b_sampled_rows_dense():
    """The row-by-row product used for sampled checks of huge systems agrees
    with a dense product on the rows it is asked for (any order, repeats)."""
    rng = np.random.default_rng(12)
    for seed, n in [(4, 9), (5, 50)]:
        rp, col, val = W.random_csr(n, 0.3, seed, symmetric=False)
        A = to_dense(rp, col, val)
        x = rng.standard_normal(n)
        rows = [n - 1, 0, n // 2, n // 2, 1]
        y = O.spmv_rows(rp, col, val[0], x, rows)
        ref = (A @ x)[rows]
        scale = (np.abs(A) @ np.abs(x))[rows]
        assert np.all(np.abs(y - ref) <= 4e-16 * 8 * scale + 1e-300), "sampled rows"


# --------------------------------------------------------------------------
# P3 -- A.1 for the variable-coefficient stencil (also pins the generator)
# --------------------------------------------------------------------------
def pin_p3_ones():
    N = 9
    rng = np.random.default_rng(5)
    kap = np.exp(rng.standard_normal(N ** 3))
    rp, col, val = W.varcoef_diffusion((N, N, N), kap)
    y = O.spmv(rp, col, val, np.ones(N ** 3))
    idx = np.arange(N ** 3)
    ix, iy, iz = idx % N, (idx // N) % N, idx // (N * N)
    nb = ((ix == 0).astype(int) + (ix == N - 1) + (iy == 0) + (iy == N - 1)
          + (iz == 0) + (iz == N - 1))
    expect = kap * nb
    rowsum_abs = O.spmv(rp, col, np.abs(val), np.ones(N ** 3))
    assert np.all(np.abs(y - expect) <= 1e-15 * 8 * rowsum_abs), "A.1 boundary law"


# --------------------------------------------------------------------------
# P4 -- CG terminates in m steps when b spans m eigenvectors
# --------------------------------------------------------------------------
def pin_p4_cg_krylov_termination():
    N = 32
    rp, col, val = W.laplacian_2d(N)
    pairs = [(1, 1), (2, 2), (3, 5), (7, 4), (11, 13)]
    lams = [laplacian_eigval_2d(N, j, k) for j, k in pairs]
    assert len(set(np.round(lams, 12))) == len(lams)
    for m in range(1, 6):
        b = sum((1.0 + 0.25 * i) * laplacian_eigvec_2d(N, *pairs[i]) for i in range(m))
        for pre in ("none", "jacobi"):
            # exact arithmetic terminates at step m; in fp64 the residual falls
            # off a cliff there (to ~1e-9 here: rounding times the spectral
            # spread), so the pin is the cliff rather than a 1e-10 test
            r = O.solve(rp, col, val, b, "cg", pre, tol=1e-7, maxit=50, history=True)
            assert r.status[0] == O.OK
            assert r.iters[0] == m, f"CG took {r.iters[0]} steps for {m} eigenvectors ({pre})"
            if m == 1:
                v, lam = laplacian_eigvec_2d(N, *pairs[0]), lams[0]
                assert _relerr(r.x[0], v / lam) <= 1e-14
            if m > 1:
                assert r.hist[0][m - 1] > 1e-2, "converged too early"


# --------------------------------------------------------------------------
# P5 -- at most n CG steps on tiny well-conditioned SPD systems, and config 1
# converges well within its number of distinct eigenvalues
# --------------------------------------------------------------------------
def pin_p5_cg_step_bound():
    rng = np.random.default_rng(3)
    for seed, n in [(4, 8), (5, 16), (6, 32)]:
        rp, col, val = W.random_csr(n, 0.3, seed, symmetric=True)
        b = rng.standard_normal(n)
        r = O.solve(rp, col, val, b, "cg", "none", tol=1e-10, maxit=10 * n)
        assert r.status[0] == O.OK and r.iters[0] <= n, f"n={n}: {r.iters[0]} steps"
    p = W.config(1)
    N = 32
    lams = {round(laplacian_eigval_2d(N, j, k), 10) for j in range(1, N + 1) for k in range(1, N + 1)}
    r = O.solve(p.row_ptr, p.col, p.values, p.b, "cg", "none", tol=1e-10, maxit=5000)
    assert r.status[0] == O.OK and r.iters[0] <= len(lams)


# --------------------------------------------------------------------------
# P6 -- forward solves against dense LU (numpy.linalg.solve)
# --------------------------------------------------------------------------
def _dense_cases():
    p1 = W.config(1, size=16)
    p2 = W.config(2, size=6)
    p3 = W.config(3, size=12, batch=3)
    p4 = W.config(4, size=16)
    return [p1, p2, p3, p4]


def pin_p6_dense_solve():
    for p in _dense_cases():
        r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, p.tol, 5000)
        for s in range(p.batch):
            A = to_dense(p.row_ptr, p.col, p.values[s])
            xd = np.linalg.solve(A, p.b[s])
            kap = np.linalg.cond(A)
            assert r.status[s] == O.OK, p.name
            assert _relerr(r.x[s], xd) <= kap * p.tol, f"{p.name} sys {s}: {_relerr(r.x[s], xd)}"


# --------------------------------------------------------------------------
# P7 -- Jacobi-PCG on a diagonal matrix converges in one step to b/d
# --------------------------------------------------------------------------
def pin_p7_jacobi_diagonal():
    n = 40
    rng = np.random.default_rng(8)
    d = rng.uniform(0.5, 20.0, n)
    rp = np.arange(n + 1, dtype=np.int32)
    col = np.arange(n, dtype=np.int32)
    b = rng.standard_normal(n)
    r = O.solve(rp, col, d[None, :], b, "cg", "jacobi", tol=1e-12, maxit=5)
    assert r.status[0] == O.OK and r.iters[0] == 1
    assert _relerr(r.x[0], b / d) <= 4e-16


# --------------------------------------------------------------------------
# P8 -- BiCGStab on an SPD matrix returns CG's solution
# --------------------------------------------------------------------------
def pin_p8_bicgstab_vs_cg():
    p = W.config(1)
    rc = O.solve(p.row_ptr, p.col, p.values, p.b, "cg", "none", 1e-12, 5000)
    rb = O.solve(p.row_ptr, p.col, p.values, p.b, "bicgstab", "none", 1e-12, 5000)
    assert rc.status[0] == O.OK and rb.status[0] == O.OK
    assert _relerr(rb.x[0], rc.x[0]) <= 1e-9


# --------------------------------------------------------------------------
# P9 -- transpose map: permutation, involution, dense transpose, <Ax,y>=<x,A^T y>
# --------------------------------------------------------------------------
def pin_p9_transpose():
    for seed, n in [(21, 9), (22, 40)]:
        rp, col, val = W.random_csr(n, 0.25, seed, symmetric=False)
        rpt, ct, perm = O.transpose(n, rp, col)
        assert np.array_equal(np.sort(perm), np.arange(col.shape[0]))
        At = to_dense(rpt, ct, val[0][perm])
        assert np.array_equal(At, to_dense(rp, col, val).T)
        rptt, ctt, permt = O.transpose(n, rpt, ct)
        assert np.array_equal(rptt, rp.astype(np.int64)) and np.array_equal(ctt, col)
        assert np.array_equal(perm[permt], np.arange(col.shape[0]))
        for i in range(n):  # sorted rows of A^T
            seg = ct[rpt[i]:rpt[i + 1]]
            assert np.all(np.diff(seg) > 0)
    p = W.config(4, size=256)
    rng = np.random.default_rng(9)
    x, y = rng.standard_normal(p.n), rng.standard_normal(p.n)
    rpt, ct, perm = O.transpose(p.n, p.row_ptr, p.col)
    lhs = O.dot(O.spmv(p.row_ptr, p.col, p.values, x), y)
    rhs = O.dot(x, O.spmv(rpt, ct, p.values[0][perm], y))
    assert abs(lhs - rhs) <= 1e-13 * abs(lhs)
    q = W.config(2, size=12)  # symmetric pattern and values
    rpt, ct, perm = O.transpose(q.n, q.row_ptr, q.col)
    assert np.array_equal(perm[perm], np.arange(q.nnz))
    assert np.array_equal(q.values[0][perm], q.values[0])


# --------------------------------------------------------------------------
# P10 -- symmetric A: the adjoint solve with g = b gives lambda = x (bitwise)
# --------------------------------------------------------------------------
def pin_p10_symmetric_adjoint():
    p = W.config(2, size=10)
    r = O.solve(p.row_ptr, p.col, p.values, p.b, "cg", "jacobi", 1e-10, 1000)
    a = O.adjoint(p.row_ptr, p.col, p.values, r.x, p.b, "cg", "jacobi", 1e-10, 1000)
    assert np.array_equal(a.grad_b, r.x)
    rb = O.solve(p.row_ptr, p.col, p.values, p.b, "bicgstab", "none", 1e-10, 1000)
    ab = O.adjoint(p.row_ptr, p.col, p.values, rb.x, p.b, "bicgstab", "none", 1e-10, 1000)
    assert np.array_equal(ab.grad_b, rb.x)


# --------------------------------------------------------------------------
# P11 -- closed-form gradient for A = diag(d), L = 0.5 ||x - x_t||^2
# --------------------------------------------------------------------------
def pin_p11_diag_gradient():
    n = 30
    rng = np.random.default_rng(12)
    d = rng.uniform(1.0, 4.0, n)
    b = rng.standard_normal(n)
    xt = rng.uniform(-1, 1, n)
    rp = np.arange(n + 1, dtype=np.int32)
    col = np.arange(n, dtype=np.int32)
    for method, pre in (("cg", "jacobi"), ("cg", "none"), ("bicgstab", "none")):
        r = O.solve(rp, col, d[None, :], b, method, pre, 1e-13, 200)
        a = O.adjoint(rp, col, d[None, :], r.x, r.x - xt, method, pre, 1e-13, 200)
        x = b / d
        assert _relerr(a.grad_values[0], -(x - xt) * b / d ** 2) <= 1e-12, method
        assert _relerr(a.grad_b[0], (x - xt) / d) <= 1e-12, method


# --------------------------------------------------------------------------
# P12 -- central finite differences of L = 0.5||x - x_t||^2 (dense LU solves)
# --------------------------------------------------------------------------
def _fd_case(p, s=0):
    A0 = to_dense(p.row_ptr, p.col, p.values[s])
    rows = pattern_rows(p.row_ptr)
    cols = np.asarray(p.col, dtype=np.int64)
    b0, xt = p.b[s].astype(np.float64), p.x_t[s].astype(np.float64)

    def L(A, b):
        x = np.linalg.solve(A, b)
        return 0.5 * float(np.dot(x - xt, x - xt))

    gv = np.empty(p.nnz)
    for k in range(p.nnz):
        v = A0[rows[k], cols[k]]
        eps = 1e-6 * max(1.0, abs(v))
        Ap, Am = A0.copy(), A0.copy()
        Ap[rows[k], cols[k]] += eps
        Am[rows[k], cols[k]] -= eps
        gv[k] = (L(Ap, b0) - L(Am, b0)) / (2 * eps)
    gb = np.empty(p.n)
    for i in range(p.n):
        eps = 1e-6 * max(1.0, abs(b0[i]))
        bp, bm = b0.copy(), b0.copy()
        bp[i] += eps
        bm[i] -= eps
        gb[i] = (L(A0, bp) - L(A0, bm)) / (2 * eps)
    return gv, gb


def pin_p12_finite_differences():
    cases = [W.config(1, size=4), W.config(2, size=2), W.config(4, size=4)]
    rp, col, val = W.random_csr(12, 0.3, 31, symmetric=False)
    rng = np.random.default_rng(31)
    cases.append(W.Problem("random_nonsym_12", 12, rp, col, val, rng.standard_normal((1, 12)),
                           rng.uniform(-1, 1, (1, 12)), method="bicgstab", precond="none",
                           tol=1e-13, maxit=500))
    for p in cases:
        r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, 1e-13, 500)
        a = O.adjoint(p.row_ptr, p.col, p.values, r.x, r.x - p.x_t, p.method, p.precond, 1e-13, 500)
        gv, gb = _fd_case(p)
        assert np.max(np.abs(a.grad_values[0] - gv)) <= 1e-6 * np.max(np.abs(gv)), p.name
        assert np.max(np.abs(a.grad_b[0] - gb)) <= 1e-6 * np.max(np.abs(gb)), p.name


# --------------------------------------------------------------------------
# P13 -- grad_values equals the dense -lambda x^T restricted to the pattern
# --------------------------------------------------------------------------
def pin_p13_dense_outer():
    p = W.config(4, size=8)
    r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, 1e-12, 1000)
    g = r.x[0] - p.x_t[0]
    a = O.adjoint(p.row_ptr, p.col, p.values, r.x, g, p.method, p.precond, 1e-12, 1000)
    A = to_dense(p.row_ptr, p.col, p.values[0])
    lam = np.linalg.solve(A.T, g)
    x = np.linalg.solve(A, p.b[0])
    full = -np.outer(lam, x)
    assert _relerr(a.grad_values[0], full[pattern_rows(p.row_ptr), p.col]) <= 1e-9
    assert _relerr(a.grad_b[0], lam) <= 1e-9


# --------------------------------------------------------------------------
# P14 -- homogeneity: sum(gradA * A) + sum(gradb * b) = lambda.(b - A x)
# (x(tA, tb) = x(A, b) for every t; derived here, not printed on the pages)
# --------------------------------------------------------------------------
def pin_p14_homogeneity():
    for p in (W.config(2, size=20), W.config(4, size=64), W.config(3, size=16, batch=2)):
        r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, p.tol, 5000)
        a = O.adjoint(p.row_ptr, p.col, p.values, r.x, r.x - p.x_t, p.method, p.precond, p.tol, 5000)
        for s in range(p.batch):
            res = p.b[s] - O.spmv(p.row_ptr, p.col, p.values[s], r.x[s])
            lhs = O.dot(a.grad_values[s], p.values[s]) + O.dot(a.grad_b[s], p.b[s])
            scale = O.dot(np.abs(a.grad_values[s]), np.abs(p.values[s]))
            assert abs(lhs - O.dot(a.grad_b[s], res)) <= 1e-13 * scale, p.name
            assert abs(lhs) <= 10 * p.tol * scale, p.name


# --------------------------------------------------------------------------
# P15 -- a batch equals the loop of its single systems (bitwise)
# --------------------------------------------------------------------------
def pin_p15_batch_is_loop():
    p = W.config(3, size=10, batch=4)
    r = O.solve(p.row_ptr, p.col, p.values, p.b, "cg", "jacobi", 1e-10, 1000)
    for s in range(p.batch):
        rs = O.solve(p.row_ptr, p.col, p.values[s], p.b[s], "cg", "jacobi", 1e-10, 1000)
        assert np.array_equal(rs.x[0], r.x[s]) and rs.iters[0] == r.iters[s]


# --------------------------------------------------------------------------
# pattern validation (invalid inputs are rejected, valid ones give diagpos)
# --------------------------------------------------------------------------
def pin_pattern_checks():
    rp, col, _ = W.laplacian_2d(5)
    st, dp = O.check_pattern(25, rp, col)
    assert st == O.OK and np.all(col[dp] == np.arange(25))
    bad = col.copy()
    bad[1], bad[2] = bad[2], bad[1]                     # unsorted row
    assert O.check_pattern(25, rp, bad)[0] == O.ERR_PATTERN
    bad = col.copy()
    bad[-1] = 25                                          # out of range
    assert O.check_pattern(25, rp, bad)[0] == O.ERR_PATTERN
    bad = col.copy()
    bad[1] = bad[0]                                       # duplicate
    assert O.check_pattern(25, rp, bad)[0] == O.ERR_PATTERN
    rp2, col2 = np.array([0, 1, 2]), np.array([1, 0], dtype=np.int32)  # no diagonal
    assert O.check_pattern(2, rp2, col2)[0] == O.ERR_PATTERN
    rp3 = rp.copy()
    rp3[3] = rp3[4] + 1                                   # decreasing row_ptr
    assert O.check_pattern(25, rp3, col)[0] == O.ERR_PATTERN


def pin_special_cases():
    p = W.config(1, size=6)
    r = O.solve(p.row_ptr, p.col, p.values, np.zeros(p.n), "cg", "jacobi", 1e-10, 100)
    assert r.status[0] == O.OK and r.iters[0] == 0 and not np.any(r.x)
    r = O.solve(p.row_ptr, p.col, p.values, np.zeros(p.n), "bicgstab", "none", 1e-10, 100)
    assert r.status[0] == O.OK and r.iters[0] == 0 and not np.any(r.x)
    r = O.solve(p.row_ptr, p.col, p.values, p.b, "cg", "none", 1e-10, 3)
    assert r.status[0] == O.NOT_CONVERGED and r.iters[0] == 3
    v = p.values.copy()
    v[0, np.asarray(O.check_pattern(p.n, p.row_ptr, p.col)[1])[0]] = 0.0
    r = O.solve(p.row_ptr, p.col, v, p.b, "cg", "jacobi", 1e-10, 100)
    assert r.status[0] == O.ERR_ZERO_DIAG
    # indefinite symmetric matrix: p.Ap <= 0 is reported as a breakdown
    rp = np.array([0, 1, 2], dtype=np.int32)
    col = np.array([0, 1], dtype=np.int32)
    r = O.solve(rp, col, np.array([[1.0, -1.0]]), np.array([0.0, 1.0]), "cg", "none", 1e-10, 10)
    assert r.status[0] == O.BREAKDOWN
    # BiCGStab breakdown: rhat.v = 0 for A = [[0,1],[1,0]], b = e1
    rp = np.array([0, 2, 4], dtype=np.int32)
    col = np.array([0, 1, 0, 1], dtype=np.int32)
    r = O.solve(rp, col, np.array([[0.0, 1.0, 1.0, 0.0]]), np.array([1.0, 0.0]), "bicgstab",
                "none", 1e-10, 10)
    assert r.status[0] == O.BREAKDOWN


# --------------------------------------------------------------------------
# Non-finite input (reading: a Krylov denominator that is zero or NaN ends
# the iteration with BREAKDOWN).  A NaN in b makes the first denominator
# NaN (CG: p.Ap; BiCGStab: rhat.r), so both stop at iteration 0 with x = 0.
# An infinite off-diagonal value A_ij turns r_i into NaN within one
# iteration (alpha = rho / inf = 0 and r_i - 0 * inf), so the next
# denominator is NaN.
# --------------------------------------------------------------------------
def pin_nonfinite_input():
    p = W.config(1, size=6)
    b = p.b.copy()
    b[0, 7] = np.nan
    for method, pre in (("cg", "jacobi"), ("cg", "none"), ("bicgstab", "none")):
        r = O.solve(p.row_ptr, p.col, p.values, b, method, pre, 1e-10, 100)
        assert r.status[0] == O.BREAKDOWN and r.iters[0] == 0, (method, pre)
        assert not np.any(r.x), (method, pre)
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    for k in np.nonzero(rows != p.col)[0][[5, 6, 11, 20]]:
        i, j = int(rows[k]), int(p.col[k])
        v = p.values.copy()
        v[0, k] = np.inf
        # BiCGStab: rhat.v = b_i * inf is infinite, alpha = 0, s_i = NaN, so
        # t.t is NaN in iteration 1: breakdown with no iteration completed
        r = O.solve(p.row_ptr, p.col, v, p.b, "bicgstab", "none", 1e-10, 100)
        assert r.status[0] == O.BREAKDOWN and r.iters[0] == 0, k
        # CG: p_0 = z_0 = b / diag(A); p.Ap holds p_i * inf * p_j, negative
        # (a breakdown at once) or positive (alpha = 0, r_i = NaN, then a NaN
        # p.Ap in iteration 2)
        r = O.solve(p.row_ptr, p.col, v, p.b, "cg", "jacobi", 1e-10, 100)
        expect = 1 if p.b[0, i] * p.b[0, j] > 0 else 0
        assert r.status[0] == O.BREAKDOWN and r.iters[0] == expect, k


# --------------------------------------------------------------------------
# P16 -- BiCGStab half step: b an eigenvector => s = 0 after one product,
# x = v / lambda (closed form), one iteration, one SpMV
# --------------------------------------------------------------------------
def pin_p16_bicgstab_half_step():
    N = 32
    rp, col, val = W.laplacian_2d(N)
    for (j, k) in [(1, 1), (5, 9)]:
        v = laplacian_eigvec_2d(N, j, k)
        lam = laplacian_eigval_2d(N, j, k)
        r = O.solve(rp, col, val, v, "bicgstab", "none", tol=1e-10, maxit=20)
        assert r.status[0] == O.OK and r.iters[0] == 1 and r.spmv[0] == 1
        assert _relerr(r.x[0], v / lam) <= 1e-13


# --------------------------------------------------------------------------
# P17 -- backward pass of the product y = A x: dense transpose product and
# the dense outer product g x^T restricted to the pattern
# --------------------------------------------------------------------------
def pin_p17_matvec_vjp_dense():
    rng = np.random.default_rng(21)
    for seed, n in [(6, 9), (7, 40)]:
        rp, col, val = W.random_csr(n, 0.25, seed, symmetric=False)
        A = to_dense(rp, col, val)
        x = rng.standard_normal(n)
        g = rng.standard_normal(n)
        gx, gv = O.matvec_vjp(rp, col, val[0], x, g)
        scale = np.abs(A).T @ np.abs(g)
        assert np.all(np.abs(gx - A.T @ g) <= 4e-16 * 8 * scale + 1e-300), "A^T g"
        rows = np.repeat(np.arange(n), np.diff(rp))
        assert np.array_equal(gv, g[rows] * x[col]), "g x^T on the pattern"


# --------------------------------------------------------------------------
# P18 -- the same backward pass by central differences of L = g . (A x)
# --------------------------------------------------------------------------
def pin_p18_matvec_vjp_finite_differences():
    rng = np.random.default_rng(22)
    rp, col, val = W.random_csr(12, 0.3, 8, symmetric=False)
    v = val[0].copy()
    x = rng.standard_normal(12)
    g = rng.standard_normal(12)
    loss = lambda vv, xx: float(g @ O.spmv(rp, col, vv, xx))
    gx, gv = O.matvec_vjp(rp, col, v, x, g)
    eps = 1e-6
    for k in range(len(v)):
        vp, vm = v.copy(), v.copy()
        vp[k] += eps
        vm[k] -= eps
        fd = (loss(vp, x) - loss(vm, x)) / (2 * eps)
        assert abs(fd - gv[k]) <= 1e-6 * max(1.0, abs(gv[k])), ("values", k)
    for j in range(12):
        xp, xm = x.copy(), x.copy()
        xp[j] += eps
        xm[j] -= eps
        fd = (loss(v, xp) - loss(v, xm)) / (2 * eps)
        assert abs(fd - gx[j]) <= 1e-6 * max(1.0, abs(gx[j])), ("x", j)


# --------------------------------------------------------------------------
# P19 -- nonlinear adjoint, c = 0: Newton is one linear solve and the
# gradients are the linear adjoint's
# --------------------------------------------------------------------------
def pin_p19_nonlinear_reduces_to_linear():
    from oracle import nonlinear as NL
    p = W.config(2, size=6)
    v = p.values[0]
    f = p.b[0]
    c = np.zeros(p.n)
    u, it, norms = NL.newton(p.row_ptr, p.col, v, c, f, tol=1e-10)
    assert it == 1 and norms[-1] <= 1e-10 * norms[0]
    g = u - p.x_t[0]
    gv, gc, gf = NL.adjoint(p.row_ptr, p.col, v, c, u, g)
    a = O.adjoint(p.row_ptr, p.col, v, u, g, "cg", "jacobi", 1e-12, 10000)
    assert _relerr(gv, a.grad_values[0]) <= 1e-9 and _relerr(gf, a.grad_b[0]) <= 1e-9


# --------------------------------------------------------------------------
# P20 -- nonlinear adjoint against central differences of a dense Newton
# (numpy.linalg.solve; a one-entry perturbation of A breaks symmetry)
# --------------------------------------------------------------------------
def _dense_newton(A, c, f):
    u = np.zeros(len(f))
    for _ in range(60):
        F = A @ u + c * u ** 3 - f
        if np.linalg.norm(F) <= 1e-15 * np.linalg.norm(f):
            break
        u = u - np.linalg.solve(A + np.diag(3.0 * c * u * u), F)
    return u


def pin_p20_nonlinear_adjoint_finite_differences():
    from oracle import nonlinear as NL
    rng = np.random.default_rng(31)
    rp, col, val = W.varcoef_diffusion((4, 4), np.exp(0.5 * rng.standard_normal(16)))
    v = val[0]
    c = rng.uniform(0.5, 2.0, 16)
    f = 3.0 * rng.standard_normal(16)
    ut = rng.standard_normal(16)
    u, it, _ = NL.newton(rp, col, v, c, f, tol=1e-14, lin_tol=1e-15)
    A = to_dense(rp, col, v)
    assert _relerr(u, _dense_newton(A, c, f)) <= 1e-12
    assert it >= 3  # the cubic term matters
    gv, gc, gf = NL.adjoint(rp, col, v, c, u, u - ut, lin_tol=1e-15)
    loss = lambda A_, c_, f_: 0.5 * np.sum((_dense_newton(A_, c_, f_) - ut) ** 2)
    eps = 1e-6
    rows = np.repeat(np.arange(16), np.diff(rp))
    for k in range(len(v)):
        Ap, Am = A.copy(), A.copy()
        Ap[rows[k], col[k]] += eps
        Am[rows[k], col[k]] -= eps
        fd = (loss(Ap, c, f) - loss(Am, c, f)) / (2 * eps)
        assert abs(fd - gv[k]) <= 1e-6 * max(1.0, abs(gv[k])), ("v", k)
    for i in range(16):
        e = np.zeros(16)
        e[i] = eps
        fd = (loss(A, c + e, f) - loss(A, c - e, f)) / (2 * eps)
        assert abs(fd - gc[i]) <= 1e-6 * max(1.0, abs(gc[i])), ("c", i)
        fd = (loss(A, c, f + e) - loss(A, c, f - e)) / (2 * eps)
        assert abs(fd - gf[i]) <= 1e-6 * max(1.0, abs(gf[i])), ("f", i)


def pin_p21_nonlinear_adjoint_nonsymmetric():
    """The same central-difference check with a nonsymmetric A (upwind
    convection-diffusion) and BiCGStab: the adjoint must use J^T."""
    from oracle import nonlinear as NL
    rng = np.random.default_rng(32)
    p = W.config(4, size=4)
    rp, col, v = p.row_ptr, p.col, p.values[0] / 19.0
    c = rng.uniform(0.5, 2.0, 16)
    f = 2.0 * rng.standard_normal(16)
    ut = rng.standard_normal(16)
    kw = dict(method="bicgstab", precond="none")
    u, it, _ = NL.newton(rp, col, v, c, f, tol=1e-14, lin_tol=1e-15, **kw)
    A = to_dense(rp, col, v)
    assert _relerr(u, _dense_newton(A, c, f)) <= 1e-12 and it >= 3
    gv, gc, gf = NL.adjoint(rp, col, v, c, u, u - ut, lin_tol=1e-15, **kw)
    loss = lambda A_, c_, f_: 0.5 * np.sum((_dense_newton(A_, c_, f_) - ut) ** 2)
    eps = 1e-6
    rows = np.repeat(np.arange(16), np.diff(rp))
    for k in range(len(v)):
        Ap, Am = A.copy(), A.copy()
        Ap[rows[k], col[k]] += eps
        Am[rows[k], col[k]] -= eps
        fd = (loss(Ap, c, f) - loss(Am, c, f)) / (2 * eps)
        assert abs(fd - gv[k]) <= 1e-6 * max(1.0, abs(gv[k])), ("v", k)
    for i in range(16):
        e = np.zeros(16)
        e[i] = eps
        fd = (loss(A, c + e, f) - loss(A, c - e, f)) / (2 * eps)
        assert abs(fd - gc[i]) <= 1e-6 * max(1.0, abs(gc[i])), ("c", i)
        fd = (loss(A, c, f + e) - loss(A, c, f - e)) / (2 * eps)
        assert abs(fd - gf[i]) <= 1e-6 * max(1.0, abs(gf[i])), ("f", i)


# --------------------------------------------------------------------------
# P22 -- eigenvalues: closed-form spectrum of the Dirichlet Laplacian
# --------------------------------------------------------------------------
def pin_p22_eigsh_laplacian_spectrum():
    from oracle import eigen as E
    N = 10
    rp, col, val = W.laplacian_2d(N)
    lam = np.sort([laplacian_eigval_2d(N, j, k) for j in range(1, N + 1)
                   for k in range(1, N + 1)])
    w, V = E.eigsh(rp, col, val[0], k=4)
    assert np.allclose(w, lam[:4], rtol=1e-13, atol=0)
    w, V = E.eigsh(rp, col, val[0], k=3, largest=True)
    assert np.allclose(w, lam[::-1][:3], rtol=1e-13, atol=0)
    # the lowest mode is the product of half sine waves
    v = laplacian_eigvec_2d(N, 1, 1)
    v = v / np.linalg.norm(v)
    assert abs(abs(float(v @ E.eigsh(rp, col, val[0], k=1)[1][0])) - 1.0) <= 1e-12


# --------------------------------------------------------------------------
# P23 -- eigenvalue gradient against central differences (perturbing one
# stored entry; eigenvalues of the perturbed matrix by numpy.linalg.eigvals)
# --------------------------------------------------------------------------
def pin_p23_eig_grad_finite_differences():
    from oracle import eigen as E
    rng = np.random.default_rng(33)
    rp, col, val = W.varcoef_diffusion((4, 4), np.exp(0.5 * rng.standard_normal(16)))
    v = val[0]
    A = E.dense(rp, col, v)
    rows = np.repeat(np.arange(16), np.diff(rp))
    for largest in (False, True):
        w, V = E.eigsh(rp, col, v, k=2, largest=largest)
        g = np.array([1.0, -0.5])
        gr = E.eig_grad(rp, col, V, g)
        eps = 1e-7
        for k in range(len(v)):
            fd = 0.0
            for q in range(2):
                vals = []
                for sgn in (1, -1):
                    Ap = A.copy()
                    Ap[rows[k], col[k]] += sgn * eps
                    ev = np.linalg.eigvals(Ap).real
                    vals.append(ev[np.argmin(np.abs(ev - w[q]))])
                fd += g[q] * (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - gr[k]) <= 1e-6 * max(1.0, abs(gr[k])), (largest, k)


ALL_PINS = [pin_p1_spmv_eigvecs, pin_p2_spmv_dense, pin_p2b_sampled_rows_dense, pin_p3_ones, pin_p4_cg_krylov_termination,
            pin_p5_cg_step_bound, pin_p6_dense_solve, pin_p7_jacobi_diagonal,
            pin_p8_bicgstab_vs_cg, pin_p9_transpose, pin_p10_symmetric_adjoint,
            pin_p11_diag_gradient, pin_p12_finite_differences, pin_p13_dense_outer,
            pin_p14_homogeneity, pin_p15_batch_is_loop, pin_p16_bicgstab_half_step,
            pin_p17_matvec_vjp_dense, pin_p18_matvec_vjp_finite_differences,
            pin_p19_nonlinear_reduces_to_linear, pin_p20_nonlinear_adjoint_finite_differences,
            pin_p21_nonlinear_adjoint_nonsymmetric, pin_p22_eigsh_laplacian_spectrum,
            pin_p23_eig_grad_finite_differences,
            pin_pattern_checks, pin_special_cases, pin_nonfinite_input]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[f.__name__ for f in ALL_PINS])
def test_pin(pin):
    pin()
