"""Second gates on the GPU's outputs, beyond element-wise parity.

  - Homogeneity (pin P14 of the oracle, evaluated on the GPU's arrays):
    x(tA, tb) = x(A, b) gives sum_k gv_k v_k + sum_i gb_i b_i = lambda.(b - A x),
    which a converged solve makes at most ||lambda|| ||b - A x||: checked
    against 10 tol ||lambda|| ||b|| plus the rounding of the two sums.
  - True residuals recomputed by the oracle: ||b - A x|| / ||b|| and
    ||g - A^T lambda|| / ||g|| (g = x - x_t) within 10 tol, configs 1-4.
  - Non-finite input (reading: a Krylov denominator that is zero or NaN is a
    breakdown): a NaN in b, or an infinite or NaN value, stops every solver
    path with the oracle's status and iteration count, and the call returns.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import banner, gpu_forward_adjoint, tdtype, to_dev

pytestmark = pytest.mark.gpu


def homogeneity(p, g, limit):
    """|sum gv v + sum gb b| <= limit ||lambda|| ||b|| + rounding, per system,
    from the device arrays (sums in fp64 on the device)."""
    d = g["dev"]
    gv = torch.from_numpy(g["gv"]).to(d["val"].device, torch.float64)
    gb = torch.from_numpy(g["gb"]).to(d["val"].device, torch.float64)
    v = d["val"].to(torch.float64).reshape(p.batch, -1)
    b = d["b"].to(torch.float64).reshape(p.batch, -1)
    gvv = gv.reshape(p.batch, -1) * v
    gbb = gb.reshape(p.batch, -1) * b
    S = gvv.sum(dim=1) + gbb.sum(dim=1)
    mag = gvv.abs().sum(dim=1) + gbb.abs().sum(dim=1)
    eps = np.finfo(p.values.dtype).eps
    bound = limit * torch.linalg.norm(gb.reshape(p.batch, -1), dim=1) * \
        torch.linalg.norm(b, dim=1) + 64 * eps * mag
    ratio = (S.abs() / bound).cpu().numpy()
    assert np.all(ratio <= 1.0), (p.name, float(ratio.max()))
    return float(ratio.max())


def true_residuals(p, g, limit, systems=None):
    """Oracle-recomputed relative residuals of x (A x = b) and of lambda
    (A^T lambda = x - x_t) for the given systems."""
    systems = range(p.batch) if systems is None else systems
    rpt, ct, perm = O.transpose(p.n, p.row_ptr, p.col)
    worst = 0.0
    for s in systems:
        v = p.values[s].astype(np.float64)
        x = g["x"][s].astype(np.float64)
        tr = O.true_relres(p.row_ptr, p.col, v, x, p.b[s].astype(np.float64))[0]
        gx = x - p.x_t[s].astype(np.float64)
        ta = O.true_relres(rpt, ct, v[perm], g["gb"][s].astype(np.float64), gx)[0]
        assert tr <= limit and ta <= limit, (p.name, s, tr, ta)
        worst = max(worst, tr, ta)
    return worst


CONFIGS = {
    "cfg1": lambda: W.config(1),
    "cfg2": lambda: W.config(2),
    "cfg3_fp64": lambda: W.config(3),
    "cfg3_fp32": lambda: W.config(3, dtype=np.float32),
    "cfg4": lambda: W.config(4),
}


@pytest.mark.parametrize("case", list(CONFIGS))
def test_homogeneity_and_true_residuals(hip, case):
    banner(f"gates {case}")
    p = CONFIGS[case]()
    g = gpu_forward_adjoint(hip, p)
    assert np.all(g["info"]["status"] == 0) and np.all(g["ainfo"]["status"] == 0)
    fp32 = p.values.dtype == np.float32
    # fp32 solves stop at 1e-5 on the fp32 recurrence; their true residual in
    # fp64 is bounded by the fp32 rounding of x as well (1e-3, as for x)
    limit = 1e-3 if fp32 else 10 * p.tol
    r = homogeneity(p, g, limit)
    systems = range(0, p.batch, max(1, p.batch // 64))
    t = true_residuals(p, g, limit, systems)
    banner(f"  homogeneity {r:.2e} of its bound, worst true residual {t:.2e}")
    g["pattern"].close()


# ------------------------------------------------------------------ non-finite input

def _nonfinite_cases(p):
    """(label, values, b) with one NaN in b, one infinite off-diagonal value,
    one NaN value."""
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    off = np.nonzero(rows != p.col)[0]
    k = int(off[len(off) // 3])
    b = p.b.copy()
    b[0, p.n // 2] = np.nan
    vi = p.values.copy()
    vi[0, k] = np.inf
    vn = p.values.copy()
    vn[0, k] = np.nan
    return [("nan_b", p.values, b), ("inf_value", vi, p.b), ("nan_value", vn, p.b)]


def _graph(method):
    from test_gpu_row_plan import directed_graph_problem, graph_problem
    return directed_graph_problem(20000, 19) if method == "bicgstab" else graph_problem(30000, 13)


PATHS = {
    "block_cg": lambda: W.config(1),
    "grid_cg_diagonal_major": lambda: W.config(2, size=20),
    "grid_bicgstab": lambda: W.config(4, size=40),
    "split_cg": lambda: _graph("cg"),
    "split_bicgstab": lambda: _graph("bicgstab"),
}


@pytest.mark.parametrize("path", list(PATHS))
def test_nonfinite_input_stops_like_the_oracle(hip, path):
    p = PATHS[path]()
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=p.method == "bicgstab")
    for label, v, b in _nonfinite_cases(p):
        banner(f"non-finite {path} {label}")
        r = O.solve(p.row_ptr, p.col, v, b, p.method, p.precond, p.tol, p.maxit)
        for kw in ({}, {"profile": True}):
            x, info = pat.solve(torch.from_numpy(v).cuda(), torch.from_numpy(b).cuda(),
                                tol=p.tol, maxit=p.maxit, method=p.method, precond=p.precond,
                                check=False, **kw)
            torch.cuda.synchronize()
            assert info["status"][0] == r.status[0] == hip.SLA_BREAKDOWN, (label, kw, info)
            assert info["iters"][0] == r.iters[0], (label, kw, info["iters"], r.iters)
            xs = x.cpu().numpy()[0]
            both = np.isfinite(xs) & np.isfinite(r.x[0])
            assert np.array_equal(np.isfinite(xs), np.isfinite(r.x[0])), (label, kw)
            assert np.allclose(xs[both], r.x[0][both], rtol=1e-12, atol=0), (label, kw)
    # the adjoint with a NaN in dL/dx
    x, info = pat.solve(d["val"], d["b"], tol=p.tol, maxit=p.maxit, method=p.method,
                        precond=p.precond)
    gx = x - d["xt"]
    gx[0, 3] = float("nan")
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, gx, tol=p.tol, maxit=p.maxit,
                                      method=p.method, precond=p.precond, check=False)
    a = O.adjoint(p.row_ptr, p.col, p.values, x.cpu().numpy(), gx.cpu().numpy(), p.method,
                  p.precond, p.tol, p.maxit)
    assert ainfo["status"][0] == a.status[0] == hip.SLA_BREAKDOWN
    assert ainfo["iters"][0] == a.iters[0]
    pat.close()
