"""Shared helpers of the GPU parity tests: move a workload to the device,
run the HIP path through the C ABI, run the oracle on the same arrays."""
import numpy as np
import torch

import oracle as O

FP_TOL = {np.dtype(np.float64): dict(spmv=1e-12, sol=1e-7),
          np.dtype(np.float32): dict(spmv=1e-5, sol=1e-3)}


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


def relerr(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def tdtype(p):
    return torch.float64 if p.values.dtype == np.float64 else torch.float32


def to_dev(p, dev="cuda:0"):
    return dict(rp=torch.from_numpy(np.ascontiguousarray(p.row_ptr)).to(dev),
                col=torch.from_numpy(np.ascontiguousarray(p.col)).to(dev),
                val=torch.from_numpy(np.ascontiguousarray(p.values)).to(dev),
                b=torch.from_numpy(np.ascontiguousarray(p.b)).to(dev),
                xt=torch.from_numpy(np.ascontiguousarray(p.x_t)).to(dev))


def spmv_bound(p, x, s, tol):
    """Componentwise bound tol * sum_j |A_ij| |x_j| for system s."""
    return tol * O.spmv(p.row_ptr, p.col, np.abs(p.values[s].astype(np.float64)),
                        np.abs(x.astype(np.float64))) + 1e-300


def gpu_forward_adjoint(sla, p, maxit=None, tol=None, **kw):
    d = to_dev(p)
    pat = sla.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p),
                      build_transpose=(p.method == "bicgstab"))
    opts = dict(tol=p.tol if tol is None else tol, maxit=p.maxit if maxit is None else maxit,
                method=p.method, precond=p.precond, **kw)
    x, info = pat.solve(d["val"], d["b"], **opts)
    g = x - d["xt"]
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, g, **opts)
    torch.cuda.synchronize()
    out = dict(x=x.cpu().numpy(), gv=gv.cpu().numpy(), gb=gb.cpu().numpy(), info=info,
               ainfo=ainfo, pattern=pat, dev=d)
    return out


def oracle_forward_adjoint(p, systems=None, maxit=None, tol=None):
    systems = list(range(p.batch)) if systems is None else list(systems)
    V = p.values[systems].astype(np.float64)
    B = p.b[systems].astype(np.float64)
    XT = p.x_t[systems].astype(np.float64)
    tol = p.tol if tol is None else tol
    maxit = p.maxit if maxit is None else maxit
    r = O.solve(p.row_ptr, p.col, V, B, p.method, p.precond, tol, maxit)
    a = O.adjoint(p.row_ptr, p.col, V, r.x, r.x - XT, p.method, p.precond, tol, maxit)
    return r, a
