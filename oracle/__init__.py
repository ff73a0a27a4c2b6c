"""Oracle for the differentiable sparse solve -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path
(``differentiable_sparse_linear_amd``) never imports, links or calls it, and
the two share no code: the only common module is ``workloads`` (seeded input
construction, no solver arithmetic).

The arithmetic lives in ``oracle.c`` (plain fp64 C, no FMA contraction,
left-to-right dot products).  This file builds it with gcc and marshals NumPy
arrays.  What it follows, from the torch-sla explainer pages (gist.science,
"Technical summary"):

* forward: x = A^-1 b by CG with a Jacobi (or no) preconditioner for SPD A, or
  by BiCGStab for nonsymmetric A (Methodology section 1 lists CG and BiCGStab;
  the Significance section names Jacobi as the native backend's preconditioner);
* backward: one adjoint solve A^T lambda = dL/dx, dL/db = lambda and
  dL/dA_ij = -lambda_i x_j on the stored pattern only (Methodology section 2,
  linear systems).  dL/db = lambda is not printed on the pages; it follows from
  the same implicit-function argument (b enters A x = b with coefficient +1);
* the differentiable product y = A x (``.matvec`` of the autograd-aware API,
  Methodology section 1) and its backward pass: grad_x = A^T dL/dy and
  dL/dA_ij = (dL/dy)_i x_j on the stored pattern;
* ``oracle.nonlinear``: Newton's method and the nonlinear adjoint for the
  semilinear model F(u) = A u + c u^3 - f (Methodology section 2, nonlinear
  systems);
* ``oracle.eigen``: dense eigenpairs of small symmetric systems and the
  eigenvalue gradient v_i v_j on the pattern (Methodology section 2,
  eigenvalue problems);
* ``oracle.inverse``: the loss, gradient and Adam trajectory of the
  inverse-coefficient experiment (Results: a coefficient recovered by
  gradient descent through the solver).

Inputs of any float dtype are promoted to fp64 (an fp32 problem is solved in
fp64 arithmetic on its fp32-rounded values); int32 row_ptr is widened to int64.
Batched calls are a loop of independent single-system calls.

Pins tying this code to something other than itself live in
``tests/test_oracle_pins.py`` (closed-form Laplacian spectra, dense solves,
finite differences, iteration-count bounds, transpose identities).  Nothing
here is "parity unpinned" except the exact iteration counts of the iterative
solvers, which depend on rounding order.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, NOT_CONVERGED, BREAKDOWN = 0, 1, 2
ERR_ARG, ERR_PATTERN, ERR_ZERO_DIAG, ERR_NO_MEMORY = -1, -2, -3, -4

_lib = None


def compile_source(src: str, out: str, extra=()) -> str:
    """gcc build of an oracle source file into a shared library (extra:
    more gcc flags, e.g. sanitizers)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


class using_library:
    """Context manager: route every call through another oracle build.

    Used by the mutation tests, which compile a deliberately broken copy of
    oracle.c and check that the pins reject it.
    """

    def __init__(self, path: str):
        self.path = path
        self.saved = None

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _configure(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    I = ctypes.c_int
    lib.orc_num_threads.restype = I
    lib.orc_set_num_threads.argtypes = [I]
    lib.orc_set_num_threads.restype = None
    lib.orc_spmv.argtypes = [I64, P, P, P, P, P]
    lib.orc_spmv.restype = None
    lib.orc_dot.argtypes = [I64, P, P]
    lib.orc_dot.restype = D
    lib.orc_check_pattern.argtypes = [I64, I64, P, P, P]
    lib.orc_check_pattern.restype = I
    lib.orc_transpose.argtypes = [I64, I64, P, P, P, P, P]
    lib.orc_transpose.restype = I
    lib.orc_cg.argtypes = [I64, P, P, P, P, P, D, I64, I, P, P, P]
    lib.orc_cg.restype = I
    lib.orc_bicgstab.argtypes = [I64, P, P, P, P, P, D, I64, P, P, P, P]
    lib.orc_bicgstab.restype = I
    lib.orc_grad_on_pattern.argtypes = [I64, P, P, P, P, P]
    lib.orc_grad_on_pattern.restype = None
    lib.orc_adjoint.argtypes = [I64, I64, P, P, P, P, P, I, I, D, I64, P, P, P, P, P]
    lib.orc_adjoint.restype = I
    lib.orc_matvec_vjp.argtypes = [I64, P, P, P, P, P, P, P]
    lib.orc_matvec_vjp.restype = None
    return lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS)."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on; the results do not
    depend on it (every dot product is summed in one fixed order)."""
    _load().orc_set_num_threads(int(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rp(row_ptr) -> np.ndarray:
    return np.ascontiguousarray(row_ptr, dtype=np.int64)


def _c(col) -> np.ndarray:
    return np.ascontiguousarray(col, dtype=np.int32)


def _f(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _batch2(a, n) -> np.ndarray:
    a = _f(a)
    return a.reshape(1, -1) if a.ndim == 1 else a


@dataclasses.dataclass
class SolveResult:
    x: np.ndarray          # [B, n] fp64
    iters: np.ndarray      # [B] int64
    spmv: np.ndarray       # [B] int64 (products with A)
    relres: np.ndarray     # [B] recurrence residual / ||b||
    status: np.ndarray     # [B] int
    hist: Optional[list] = None


@dataclasses.dataclass
class AdjointResult:
    grad_values: np.ndarray  # [B, nnz]
    grad_b: np.ndarray       # [B, n] (= lambda)
    iters: np.ndarray
    spmv: np.ndarray
    relres: np.ndarray
    status: np.ndarray


def spmv(row_ptr, col, values, x) -> np.ndarray:
    """y = A x for one system (1-D) or a batch sharing the pattern (2-D)."""
    lib = _load()
    rp, c = _rp(row_ptr), _c(col)
    n = rp.shape[0] - 1
    one = np.ndim(x) == 1
    V = _batch2(values, c.shape[0])
    X = _batch2(x, n)
    B = max(V.shape[0], X.shape[0])
    Y = np.empty((B, n))
    for s in range(B):
        v = V[s if V.shape[0] > 1 else 0]
        xs = X[s if X.shape[0] > 1 else 0]
        lib.orc_spmv(n, _p(rp), _p(c), _p(v), _p(xs), _p(Y[s]))
    return Y[0] if one else Y


def spmv_rows(row_ptr, col, values, x, rows) -> np.ndarray:
    """(A x)_i for the listed rows only, in fp64, each row summed in stored
    entry order -- the product's definition written out row by row, for
    sampled checks of systems too large to recompute whole.  ``values`` and
    ``x`` are 1-D (one system)."""
    rp = np.asarray(row_ptr)
    out = np.empty(len(rows))
    for j, i in enumerate(rows):
        lo, hi = int(rp[i]), int(rp[i + 1])
        vs = np.asarray(values[lo:hi], dtype=np.float64)
        xs = np.asarray(x, dtype=np.float64)[np.asarray(col[lo:hi], dtype=np.int64)]
        acc = 0.0
        for k in range(hi - lo):
            acc += float(vs[k]) * float(xs[k])
        out[j] = acc
    return out


def dot(a, b) -> float:
    a, b = _f(a), _f(b)
    return float(_load().orc_dot(a.shape[0], _p(a), _p(b)))


def check_pattern(n, row_ptr, col):
    """(status, diagpos[n]) -- status 0 or ERR_PATTERN."""
    rp, c = _rp(row_ptr), _c(col)
    dp = np.full(n, -1, dtype=np.int64)
    st = _load().orc_check_pattern(n, c.shape[0], _p(rp), _p(c), _p(dp))
    return int(st), dp


def transpose(n, row_ptr, col):
    """(row_ptr_t int64[n+1], col_t int32[nnz], perm int64[nnz])."""
    rp, c = _rp(row_ptr), _c(col)
    nnz = c.shape[0]
    rpt = np.empty(n + 1, dtype=np.int64)
    ct = np.empty(nnz, dtype=np.int32)
    perm = np.empty(nnz, dtype=np.int64)
    st = _load().orc_transpose(n, nnz, _p(rp), _p(c), _p(rpt), _p(ct), _p(perm))
    if st != OK:
        raise MemoryError("oracle transpose failed")
    return rpt, ct, perm


def solve(row_ptr, col, values, b, method: str = "cg", precond: str = "jacobi",
          tol: float = 1e-10, maxit: int = 1000, history: bool = False) -> SolveResult:
    """Forward solve of every system in the batch, system by system."""
    lib = _load()
    rp, c = _rp(row_ptr), _c(col)
    n = rp.shape[0] - 1
    V = _batch2(values, c.shape[0])
    Bm = _batch2(b, n)
    B = max(V.shape[0], Bm.shape[0])
    X = np.zeros((B, n))
    iters = np.zeros(B, dtype=np.int64)
    nmv = np.zeros(B, dtype=np.int64)
    rel = np.zeros(B)
    st = np.zeros(B, dtype=np.int64)
    hists = [] if history else None
    for s in range(B):
        v = V[s if V.shape[0] > 1 else 0]
        bs = Bm[s if Bm.shape[0] > 1 else 0]
        it = ctypes.c_int64(0)
        mv = ctypes.c_int64(0)
        rr = ctypes.c_double(0.0)
        h = np.zeros(maxit + 2) if history else None
        if method == "cg":
            code = lib.orc_cg(n, _p(rp), _p(c), _p(v), _p(bs), _p(X[s]), tol, maxit,
                              1 if precond == "jacobi" else 0, ctypes.byref(it),
                              ctypes.byref(rr), _p(h))
            mv.value = it.value
        elif method == "bicgstab":
            if precond != "none":
                raise ValueError("the oracle's BiCGStab is unpreconditioned")
            code = lib.orc_bicgstab(n, _p(rp), _p(c), _p(v), _p(bs), _p(X[s]), tol, maxit,
                                    ctypes.byref(it), ctypes.byref(mv), ctypes.byref(rr), _p(h))
        else:
            raise ValueError(method)
        iters[s], nmv[s], rel[s], st[s] = it.value, mv.value, rr.value, code
        if history:
            hists.append(h[: it.value + 1].copy())
    return SolveResult(X, iters, nmv, rel, st, hists)


def grad_on_pattern(row_ptr, col, lam, x) -> np.ndarray:
    """grad_values[s, k] = -lam[s, row(k)] * x[s, col(k)]."""
    lib = _load()
    rp, c = _rp(row_ptr), _c(col)
    n = rp.shape[0] - 1
    L = _batch2(lam, n)
    X = _batch2(x, n)
    G = np.empty((L.shape[0], c.shape[0]))
    for s in range(L.shape[0]):
        lib.orc_grad_on_pattern(n, _p(rp), _p(c), _p(L[s]), _p(X[s]), _p(G[s]))
    return G


def matvec_vjp(row_ptr, col, values, x, grad_y):
    """Backward pass of y = A x for upstream gradient grad_y = dL/dy:
    (grad_x = A^T grad_y, grad_values[k] = grad_y[row(k)] x[col(k)]), each
    [B, n] / [B, nnz] (1-D in, 1-D out)."""
    lib = _load()
    rp, c = _rp(row_ptr), _c(col)
    n = rp.shape[0] - 1
    one = np.ndim(x) == 1 and np.ndim(grad_y) == 1 and np.ndim(values) == 1
    V = _batch2(values, c.shape[0])
    X = _batch2(x, n)
    G = _batch2(grad_y, n)
    B = max(V.shape[0], X.shape[0], G.shape[0])
    gx = np.empty((B, n))
    gv = np.empty((B, c.shape[0]))
    for s in range(B):
        lib.orc_matvec_vjp(n, _p(rp), _p(c), _p(V[s if V.shape[0] > 1 else 0]),
                           _p(X[s if X.shape[0] > 1 else 0]), _p(G[s if G.shape[0] > 1 else 0]),
                           _p(gx[s]), _p(gv[s]))
    return (gx[0], gv[0]) if one else (gx, gv)


def adjoint(row_ptr, col, values, x, grad_x, method: str = "cg",
            precond: str = "jacobi", tol: float = 1e-10, maxit: int = 1000) -> AdjointResult:
    """Backward pass of x = A^-1 b for upstream gradient grad_x = dL/dx."""
    lib = _load()
    rp, c = _rp(row_ptr), _c(col)
    n = rp.shape[0] - 1
    nnz = c.shape[0]
    V = _batch2(values, nnz)
    X = _batch2(x, n)
    G = _batch2(grad_x, n)
    B = X.shape[0]
    gv = np.zeros((B, nnz))
    gb = np.zeros((B, n))
    iters = np.zeros(B, dtype=np.int64)
    nmv = np.zeros(B, dtype=np.int64)
    rel = np.zeros(B)
    st = np.zeros(B, dtype=np.int64)
    m = {"cg": 0, "bicgstab": 1}[method]
    for s in range(B):
        it = ctypes.c_int64(0)
        mv = ctypes.c_int64(0)
        rr = ctypes.c_double(0.0)
        v = V[s if V.shape[0] > 1 else 0]
        code = lib.orc_adjoint(n, nnz, _p(rp), _p(c), _p(v), _p(X[s]), _p(G[s]), m,
                               1 if precond == "jacobi" else 0, tol, maxit,
                               _p(gb[s]), _p(gv[s]), ctypes.byref(it), ctypes.byref(mv),
                               ctypes.byref(rr))
        iters[s], nmv[s], rel[s], st[s] = it.value, mv.value, rr.value, code
    return AdjointResult(gv, gb, iters, nmv, rel, st)


def true_relres(row_ptr, col, values, x, b) -> np.ndarray:
    """||b - A x|| / ||b|| per system, recomputed in fp64."""
    Ax = spmv(row_ptr, col, values, _batch2(x, _rp(row_ptr).shape[0] - 1))
    Bm = _batch2(b, Ax.shape[-1])
    R = Bm - Ax
    out = []
    for s in range(R.shape[0]):
        bn = np.sqrt(dot(Bm[s], Bm[s]))
        out.append(np.sqrt(dot(R[s], R[s])) / bn if bn > 0 else 0.0)
    return np.asarray(out)
