"""Differentiable sparse linear solves on MI355X (gfx950).

Thin Python binding over ``libsla.so`` (C ABI declared in ``include/sla.h``).
Every step of the solve runs in the library's HIP kernels; this module only
marshals torch tensors (device memory, the current stream) into the C calls,
and fails loudly if the library has not been built.

What is computed (torch-sla explainer pages on gist.science, "Technical
summary"): x = A^-1 b for CSR A by Jacobi-preconditioned CG or BiCGStab
(Methodology section 1), and the adjoint backward pass A^T lambda = dL/dx,
dL/db = lambda, dL/dA_ij = -lambda_i x_j on the stored pattern
(Methodology section 2, linear systems).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = [
    "load", "SlaError", "Pattern", "PatternList", "SparseSolve", "sparse_solve",
    "SparseMatvec", "sparse_matvec", "SparseEigsh", "sparse_eigsh",
    "sla_create", "sla_destroy", "sla_matvec", "sla_matvec_adjoint", "sla_solve",
    "sla_solve_adjoint", "sla_eigsh", "sla_eigsh_adjoint", "sla_solve_noalloc", "solve_noalloc",
    "sla_export_pattern", "sla_workspace_bytes", "sla_status_string",
    "SLA_OK", "SLA_NOT_CONVERGED", "SLA_BREAKDOWN", "SLA_ERR_ARG", "SLA_ERR_PATTERN",
    "SLA_ERR_ZERO_DIAG", "SLA_ERR_NO_MEMORY", "SLA_ERR_DEVICE", "SLA_ERR_TOO_LARGE",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsla.so")

SLA_F32, SLA_F64 = 0, 1
SLA_I32, SLA_I64 = 0, 1
SLA_CG, SLA_BICGSTAB = 0, 1
SLA_PRECOND_NONE, SLA_PRECOND_JACOBI = 0, 1
SLA_CREATE_TRANSPOSE, SLA_CREATE_WIDE_COLUMNS, SLA_CREATE_CSR_VALUES = 1, 2, 4
SLA_OK, SLA_NOT_CONVERGED, SLA_BREAKDOWN = 0, 1, 2
SLA_ERR_ARG, SLA_ERR_PATTERN, SLA_ERR_ZERO_DIAG = -1, -2, -3
SLA_ERR_NO_MEMORY, SLA_ERR_DEVICE, SLA_ERR_TOO_LARGE = -4, -5, -6

EXPORTED_SYMBOLS = ("sla_create", "sla_destroy", "sla_matvec", "sla_matvec_adjoint", "sla_solve",
                    "sla_solve_adjoint", "sla_eigsh", "sla_eigsh_adjoint", "sla_column_mode",
                    "sla_iteration_form", "sla_export_pattern", "sla_workspace_bytes", "sla_status_string",
                    "sla_last_error", "sla_solve_noalloc")

_METHODS = {"cg": SLA_CG, "bicgstab": SLA_BICGSTAB}
_PRECONDS = {"none": SLA_PRECOND_NONE, "jacobi": SLA_PRECOND_JACOBI}


class _EigOpts(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("largest", ctypes.c_int32), ("ncv", ctypes.c_int32),
                ("max_restarts", ctypes.c_int32), ("tol", ctypes.c_double)]


class _Opts(ctypes.Structure):
    _fields_ = [("tol", ctypes.c_double), ("maxit", ctypes.c_int32), ("method", ctypes.c_int32),
                ("precond", ctypes.c_int32), ("use_x0", ctypes.c_int32),
                ("graph_chunk", ctypes.c_int32), ("profile", ctypes.c_int32)]


class _Info(ctypes.Structure):
    _fields_ = [("iters", ctypes.c_void_p), ("spmv", ctypes.c_void_p), ("relres", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("kernel_ms", ctypes.c_double),
                ("kernel_launches", ctypes.c_int64), ("form", ctypes.c_int32)]


_FORMS = ("wide", "tile16", "diagonal", "diagonal-major", "diagonal-major-symmetric")


def _form_name(code: int) -> str:
    """Name of an sla_solve_info.form code ("block": the one-workgroup solver)."""
    return "block" if code < 0 else _FORMS[code]


_lib = None


def load(path: Optional[str] = None):
    """Load libsla.so (built by ``python -m differentiable_sparse_linear_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m differentiable_sparse_linear_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.sla_create.argtypes = [ctypes.POINTER(P), I64, I64, I64, I32, I32, P, P, I32, P]
    lib.sla_create.restype = I32
    lib.sla_destroy.argtypes = [P]
    lib.sla_destroy.restype = I32
    lib.sla_matvec.argtypes = [P, P, P, P, I32, P]
    lib.sla_matvec.restype = I32
    lib.sla_solve.argtypes = [P, P, P, P, ctypes.POINTER(_Opts), ctypes.POINTER(_Info), P]
    lib.sla_solve.restype = I32
    lib.sla_solve_adjoint.argtypes = [P, P, P, P, P, P, ctypes.POINTER(_Opts),
                                      ctypes.POINTER(_Info), P]
    lib.sla_solve_adjoint.restype = I32
    lib.sla_matvec_adjoint.argtypes = [P, P, P, P, P, P, P]
    lib.sla_matvec_adjoint.restype = I32
    lib.sla_eigsh.argtypes = [P, P, P, P, ctypes.POINTER(_EigOpts), P, P]
    lib.sla_eigsh.restype = I32
    lib.sla_eigsh_adjoint.argtypes = [P, P, P, I32, P, P]
    lib.sla_eigsh_adjoint.restype = I32
    lib.sla_column_mode.argtypes = [P, I32]
    lib.sla_column_mode.restype = I32
    lib.sla_iteration_form.argtypes = [P, I32]
    lib.sla_iteration_form.restype = I32
    lib.sla_export_pattern.argtypes = [P, P, P, P, P, P]
    lib.sla_export_pattern.restype = I32
    lib.sla_workspace_bytes.argtypes = [P]
    lib.sla_workspace_bytes.restype = I64
    lib.sla_status_string.argtypes = [I32]
    lib.sla_status_string.restype = ctypes.c_char_p
    lib.sla_last_error.argtypes = []
    lib.sla_last_error.restype = ctypes.c_char_p
    lib.sla_solve_noalloc.argtypes = [I64, I64, I64, I32, I32, P, P, P, P, P,
                                      ctypes.POINTER(_Opts), ctypes.POINTER(_Info), P]
    lib.sla_solve_noalloc.restype = I32
    _lib = lib
    return lib


class SlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.sla_status_string(status).decode()
        if status == SLA_ERR_DEVICE:
            msg += f" ({lib.sla_last_error().decode()})"
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def sla_status_string(status: int) -> str:
    return load().sla_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t: torch.Tensor, name: str, dtype=None, numel=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


# -------------------------------------------------------------- raw C calls

def sla_create(n, nnz, batch, dtype, row_ptr: torch.Tensor, col: torch.Tensor,
               flags: int, stream=None) -> int:
    lib = load()
    h = ctypes.c_void_p()
    itype = SLA_I64 if row_ptr.dtype == torch.int64 else SLA_I32
    dt = SLA_F64 if dtype == torch.float64 else SLA_F32
    st = lib.sla_create(ctypes.byref(h), int(n), int(nnz), int(batch), dt, itype, _ptr(row_ptr),
                        _ptr(col), int(flags), _stream(stream))
    if st != SLA_OK:
        raise SlaError(st, "sla_create")
    return h.value


def sla_destroy(h: int) -> None:
    st = load().sla_destroy(ctypes.c_void_p(h))
    if st != SLA_OK:
        raise SlaError(st, "sla_destroy")


def sla_matvec(h, values, x, y, transpose=False, stream=None) -> int:
    return load().sla_matvec(ctypes.c_void_p(h), _ptr(values), _ptr(x), _ptr(y),
                             1 if transpose else 0, _stream(stream))


def sla_matvec_adjoint(h, values, x, grad_y, grad_x, grad_values, stream=None) -> int:
    return load().sla_matvec_adjoint(ctypes.c_void_p(h), _ptr(values), _ptr(x), _ptr(grad_y),
                                     _ptr(grad_x), _ptr(grad_values), _stream(stream))


def sla_eigsh(h, values, evals: np.ndarray, evecs, opts: "_EigOpts", restarts: np.ndarray,
              stream=None) -> int:
    return load().sla_eigsh(ctypes.c_void_p(h), _ptr(values), evals.ctypes.data_as(ctypes.c_void_p),
                            _ptr(evecs), ctypes.byref(opts),
                            restarts.ctypes.data_as(ctypes.c_void_p), _stream(stream))


def sla_eigsh_adjoint(h, evecs, grad_evals, k, grad_values, stream=None) -> int:
    return load().sla_eigsh_adjoint(ctypes.c_void_p(h), _ptr(evecs), _ptr(grad_evals), int(k),
                                    _ptr(grad_values), _stream(stream))


def _make_opts(tol, maxit, method, precond, use_x0, graph_chunk, profile):
    return _Opts(float(tol), int(maxit), _METHODS[method], _PRECONDS[precond], int(use_x0),
                 int(graph_chunk), int(profile))


def _make_info(batch):
    arrs = {"iters": np.zeros(batch, np.int32), "spmv": np.zeros(batch, np.int32),
            "relres": np.zeros(batch, np.float64), "status": np.zeros(batch, np.int32)}
    info = _Info(arrs["iters"].ctypes.data, arrs["spmv"].ctypes.data, arrs["relres"].ctypes.data,
                 arrs["status"].ctypes.data, 0.0, 0)
    return info, arrs


def sla_solve(h, values, b, x, opts: _Opts, info: _Info, stream=None) -> int:
    return load().sla_solve(ctypes.c_void_p(h), _ptr(values), _ptr(b), _ptr(x), ctypes.byref(opts),
                            ctypes.byref(info), _stream(stream))


def sla_solve_adjoint(h, values, x, grad_x, grad_values, grad_b, opts: _Opts, info: _Info,
                      stream=None) -> int:
    return load().sla_solve_adjoint(ctypes.c_void_p(h), _ptr(values), _ptr(x), _ptr(grad_x),
                                    _ptr(grad_values), _ptr(grad_b), ctypes.byref(opts),
                                    ctypes.byref(info), _stream(stream))


def sla_solve_noalloc(n, nnz, batch, dtype, row_ptr, col, values, b, x, opts: _Opts,
                      info: _Info, stream=None) -> int:
    itype = SLA_I64 if row_ptr.dtype == torch.int64 else SLA_I32
    dt = SLA_F64 if dtype == torch.float64 else SLA_F32
    return load().sla_solve_noalloc(int(n), int(nnz), int(batch), dt, itype, _ptr(row_ptr),
                                    _ptr(col), _ptr(values), _ptr(b), _ptr(x), ctypes.byref(opts),
                                    ctypes.byref(info), _stream(stream))


def solve_noalloc(row_ptr: torch.Tensor, col: torch.Tensor, values: torch.Tensor,
                  b: torch.Tensor, x: torch.Tensor, tol=1e-10, maxit=1000, precond="jacobi",
                  use_x0=False, check=True, stream=None):
    """CG through sla_solve_noalloc into the caller's x (n <= 4096, batch <=
    65535; nothing is allocated on the device).  values [batch, nnz] and b, x
    [batch, n] of one float type.  Returns info as Pattern.solve does."""
    _check(row_ptr, "row_ptr")
    _check(col, "col", torch.int32)
    n, nnz = row_ptr.numel() - 1, col.numel()
    batch = b.numel() // n if n > 0 else 0
    _check(values, "values", b.dtype, batch * nnz)
    _check(b, "b", None, batch * n)
    _check(x, "x", b.dtype, batch * n)
    opts = _make_opts(tol, maxit, "cg", precond, use_x0, 0, 0)
    info, arrs = _make_info(batch)
    st = sla_solve_noalloc(n, nnz, batch, b.dtype, row_ptr, col, values, b, x, opts, info, stream)
    arrs["return"] = st
    arrs["form"] = _form_name(info.form)
    if check and st < 0:
        raise SlaError(st, "sla_solve_noalloc")
    return arrs


def sla_export_pattern(h, diagpos=None, row_ptr_t=None, col_t=None, perm=None, stream=None) -> int:
    return load().sla_export_pattern(ctypes.c_void_p(h), _ptr(diagpos), _ptr(row_ptr_t),
                                     _ptr(col_t), _ptr(perm), _stream(stream))


def sla_workspace_bytes(h) -> int:
    return int(load().sla_workspace_bytes(ctypes.c_void_p(h)))


# -------------------------------------------------------------- object API

class Pattern:
    """A CSR pattern on the device shared by ``batch`` value arrays.

    row_ptr: int32/int64 [n+1], col: int32 [nnz] (device tensors, kept alive
    by this object because the library borrows them).  ``build_transpose``
    builds the map of A^T (transposed products, BiCGStab adjoint);
    ``compact_columns`` lets the handle read a 2-byte tile-relative copy of
    the columns where every entry fits, or one 16-bit diagonal mask per row
    for stencil patterns (identical results, fewer bytes);
    ``diagonal_major`` (with compact columns) lets the solver iterations of
    3-, 5- and 7-diagonal patterns read a diagonal-major copy of the values
    made at the start of each solve (no row pointers or columns read).
    """

    def __init__(self, row_ptr: torch.Tensor, col: torch.Tensor, batch: int = 1,
                 dtype: torch.dtype = torch.float64, build_transpose: bool = False,
                 compact_columns: bool = True, stream=None, diagonal_major: bool = True):
        _check(row_ptr, "row_ptr")
        _check(col, "col", torch.int32)
        if row_ptr.dtype not in (torch.int32, torch.int64):
            raise ValueError("row_ptr must be int32 or int64")
        if dtype not in (torch.float32, torch.float64):
            raise ValueError("dtype must be float32 or float64")
        self.row_ptr, self.col = row_ptr, col
        self.n = row_ptr.numel() - 1
        self.nnz = col.numel()
        self.batch = int(batch)
        self.dtype = dtype
        self.has_transpose = bool(build_transpose)
        self.device = row_ptr.device
        flags = (SLA_CREATE_TRANSPOSE if build_transpose else 0) | \
            (0 if compact_columns else SLA_CREATE_WIDE_COLUMNS) | \
            (0 if diagonal_major else SLA_CREATE_CSR_VALUES)
        self.handle = sla_create(self.n, self.nnz, self.batch, dtype, row_ptr, col, flags, stream)

    def close(self):
        if getattr(self, "handle", None):
            sla_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self) -> int:
        return sla_workspace_bytes(self.handle)

    def column_mode(self, transpose: bool = False) -> str:
        """How the products read the columns: "wide" (int32), "tile16"
        (2 bytes per entry) or "diagonal" (a 16-bit mask per row)."""
        m = load().sla_column_mode(ctypes.c_void_p(self.handle), 1 if transpose else 0)
        if m < 0:
            raise SlaError(SLA_ERR_ARG, "sla_column_mode")
        return ("wide", "tile16", "diagonal")[m]

    def iteration_form(self, transpose: bool = False) -> str:
        """What the solver iterations read: a column mode, or
        "diagonal-major" (values repacked per solve, no index)."""
        m = load().sla_iteration_form(ctypes.c_void_p(self.handle), 1 if transpose else 0)
        if m < 0:
            raise SlaError(SLA_ERR_ARG, "sla_iteration_form")
        return ("wide", "tile16", "diagonal", "diagonal-major")[m]

    def _vals(self, values):
        _check(values, "values", self.dtype, self.batch * self.nnz)

    def _vec(self, v, name):
        _check(v, name, self.dtype, self.batch * self.n)

    def matvec(self, values, x, transpose=False, out=None, stream=None):
        self._vals(values)
        self._vec(x, "x")
        y = out if out is not None else torch.empty_like(x)
        self._vec(y, "out")
        st = sla_matvec(self.handle, values, x, y, transpose, stream)
        if st != SLA_OK:
            raise SlaError(st, "sla_matvec")
        return y

    def matvec_adjoint(self, values, x, grad_y, need_grad_x=True, need_grad_values=True,
                       stream=None):
        """Backward pass of y = A x: (grad_values, grad_x), either None when
        not asked for.  grad_x = A^T grad_y needs the transpose map."""
        self._vals(values)
        self._vec(grad_y, "grad_y")
        if need_grad_values:
            self._vec(x, "x")
        gx = torch.empty_like(grad_y) if need_grad_x else None
        gv = torch.empty_like(values) if need_grad_values else None
        st = sla_matvec_adjoint(self.handle, values, x if need_grad_values else None, grad_y,
                                gx, gv, stream)
        if st != SLA_OK:
            raise SlaError(st, "sla_matvec_adjoint")
        return gv, gx

    def eigsh(self, values, k=1, largest=False, tol=1e-10, ncv=0, max_restarts=50, check=True,
              stream=None):
        """Extreme eigenpairs of each (symmetric) system: (evals [batch, k]
        on the values' device, evecs [batch, k, n], info with the restarts
        and the return status)."""
        self._vals(values)
        evals = np.zeros((self.batch, k), dtype=np.float64)
        restarts = np.zeros(self.batch, dtype=np.int32)
        evecs = torch.empty((self.batch, k, self.n), dtype=self.dtype, device=self.device)
        opts = _EigOpts(int(k), 1 if largest else 0, int(ncv), int(max_restarts), float(tol))
        st = sla_eigsh(self.handle, values, evals, evecs, opts, restarts, stream)
        if check and st < 0:
            raise SlaError(st, "sla_eigsh")
        ev = torch.from_numpy(evals).to(device=self.device, dtype=self.dtype)
        return ev, evecs, {"restarts": restarts, "return": st}

    def eigsh_adjoint(self, evecs, grad_evals, stream=None):
        """grad_values[s, k'] = sum_q grad_evals[s, q] v_q[row(k')] v_q[col(k')]."""
        k = evecs.shape[-2]
        _check(evecs, "evecs", self.dtype, self.batch * k * self.n)
        _check(grad_evals, "grad_evals", self.dtype, self.batch * k)
        gv = torch.empty(self.batch * self.nnz, dtype=self.dtype, device=self.device)
        st = sla_eigsh_adjoint(self.handle, evecs, grad_evals, k, gv, stream)
        if st != SLA_OK:
            raise SlaError(st, "sla_eigsh_adjoint")
        return gv

    def solve(self, values, b, tol=1e-10, maxit=1000, method="cg", precond="jacobi", x0=None,
              graph_chunk=0, profile=False, check=True, out=None, stream=None):
        """Returns (x, info); info holds per-system iters/spmv/relres/status."""
        self._vals(values)
        self._vec(b, "b")
        if x0 is not None:
            self._vec(x0, "x0")
            x = x0.clone() if out is None else out.copy_(x0)
        else:
            x = out if out is not None else torch.empty_like(b)
        self._vec(x, "x")
        opts = _make_opts(tol, maxit, method, precond, x0 is not None, graph_chunk, profile)
        info, arrs = _make_info(self.batch)
        st = sla_solve(self.handle, values, b, x, opts, info, stream)
        arrs["return"] = st
        arrs["kernel_ms"] = info.kernel_ms
        arrs["kernel_launches"] = info.kernel_launches
        arrs["form"] = _form_name(info.form)
        if check and st < 0:
            raise SlaError(st, "sla_solve")
        return x, arrs

    def solve_adjoint(self, values, x, grad_x, tol=1e-10, maxit=1000, method="cg",
                      precond="jacobi", graph_chunk=0, profile=False, check=True, out=None,
                      stream=None):
        """Returns (grad_values, grad_b, info)."""
        self._vals(values)
        self._vec(x, "x")
        self._vec(grad_x, "grad_x")
        gv = torch.empty_like(values) if out is None else out[0]
        gb = torch.empty_like(grad_x) if out is None else out[1]
        opts = _make_opts(tol, maxit, method, precond, 0, graph_chunk, profile)
        info, arrs = _make_info(self.batch)
        st = sla_solve_adjoint(self.handle, values, x, grad_x, gv, gb, opts, info, stream)
        arrs["return"] = st
        arrs["kernel_ms"] = info.kernel_ms
        arrs["kernel_launches"] = info.kernel_launches
        arrs["form"] = _form_name(info.form)
        if check and st < 0:
            raise SlaError(st, "sla_solve_adjoint")
        return gv, gb, arrs

    def export_pattern(self, stream=None):
        """Derived structures: diagpos, and (row_ptr_t, col_t, perm) if built."""
        idt = self.row_ptr.dtype
        dp = torch.empty(self.n, dtype=idt, device=self.device)
        rpt = ct = pm = None
        if self.has_transpose:
            rpt = torch.empty(self.n + 1, dtype=idt, device=self.device)
            ct = torch.empty(self.nnz, dtype=torch.int32, device=self.device)
            pm = torch.empty(self.nnz, dtype=torch.int32, device=self.device)
        st = sla_export_pattern(self.handle, dp, rpt, ct, pm, stream)
        if st != SLA_OK:
            raise SlaError(st, "sla_export_pattern")
        return dp, rpt, ct, pm


class SparseSolve(torch.autograd.Function):
    """x = A^-1 b with the adjoint backward; saves only x (O(n) per system)."""

    @staticmethod
    def forward(ctx, values, b, pattern: Pattern, opts: dict):
        x, info = pattern.solve(values.contiguous(), b.contiguous(), **opts)
        ctx.pattern = pattern
        ctx.opts = opts
        ctx.save_for_backward(values, x)
        return x

    @staticmethod
    def backward(ctx, grad_x):
        values, x = ctx.saved_tensors
        gv, gb, _ = ctx.pattern.solve_adjoint(values.contiguous(), x, grad_x.contiguous(),
                                              **{k: v for k, v in ctx.opts.items()
                                                 if k not in ("x0",)})
        return gv, gb, None, None


def sparse_solve(pattern: Pattern, values: torch.Tensor, b: torch.Tensor, **opts) -> torch.Tensor:
    """Differentiable x = A(values)^-1 b; gradients flow to values and b."""
    return SparseSolve.apply(values, b, pattern, opts)


class SparseMatvec(torch.autograd.Function):
    """y = A(values) x with the product's backward pass (grad_x = A^T g needs
    a pattern built with the transpose map)."""

    @staticmethod
    def forward(ctx, values, x, pattern: Pattern):
        values, x = values.contiguous(), x.contiguous()
        ctx.pattern = pattern
        ctx.save_for_backward(values, x)
        return pattern.matvec(values, x)

    @staticmethod
    def backward(ctx, grad_y):
        values, x = ctx.saved_tensors
        gv, gx = ctx.pattern.matvec_adjoint(values, x, grad_y.contiguous(),
                                            need_grad_x=ctx.needs_input_grad[1],
                                            need_grad_values=ctx.needs_input_grad[0])
        return gv, gx, None


def sparse_matvec(pattern: Pattern, values: torch.Tensor, x: torch.Tensor) -> torch.Tensor:
    """Differentiable y = A(values) x; gradients flow to values and x."""
    return SparseMatvec.apply(values, x, pattern)


class PatternList:
    """Systems with distinct patterns (one handle per pattern), the ragged
    counterpart of the shared-pattern batch.  Each call runs pattern by
    pattern on the same stream; every product and solve runs in the
    library's kernels."""

    def __init__(self, patterns, dtype: torch.dtype = torch.float64,
                 build_transpose: bool = False, compact_columns: bool = True, stream=None):
        self.items = [Pattern(rp, col, 1, dtype, build_transpose, compact_columns, stream)
                      for rp, col in patterns]

    def __len__(self):
        return len(self.items)

    def __getitem__(self, i) -> Pattern:
        return self.items[i]

    def close(self):
        for p in self.items:
            p.close()

    def matvec(self, values, xs, transpose=False, stream=None):
        return [p.matvec(v, x, transpose=transpose, stream=stream)
                for p, v, x in zip(self.items, values, xs)]

    def solve(self, values, bs, **opts):
        """Returns a list of (x, info)."""
        return [p.solve(v, b, **opts) for p, v, b in zip(self.items, values, bs)]

    def solve_adjoint(self, values, xs, grads, **opts):
        """Returns a list of (grad_values, grad_b, info)."""
        return [p.solve_adjoint(v, x, g, **opts)
                for p, v, x, g in zip(self.items, values, xs, grads)]


class SparseEigsh(torch.autograd.Function):
    """Extreme eigenvalues of A(values) with the Hellmann-Feynman backward
    (dlambda/dA_ij = v_i v_j on the pattern, simple eigenvalues); the
    eigenvectors are returned but carry no gradient."""

    @staticmethod
    def forward(ctx, values, pattern: Pattern, opts: dict):
        evals, evecs, info = pattern.eigsh(values.contiguous(), **opts)
        ctx.pattern = pattern
        ctx.save_for_backward(evecs)
        ctx.mark_non_differentiable(evecs)
        return evals, evecs

    @staticmethod
    def backward(ctx, grad_evals, grad_evecs):
        (evecs,) = ctx.saved_tensors
        gv = ctx.pattern.eigsh_adjoint(evecs, grad_evals.contiguous())
        return gv, None, None


def sparse_eigsh(pattern: Pattern, values: torch.Tensor, **opts):
    """(evals, evecs) of A(values); evals are differentiable in values."""
    return SparseEigsh.apply(values, pattern, opts)
