"""Batches of systems too large for the one-workgroup solver (n > 4096).

CG and BiCGStab advance a group of min(batch, 65535, 2^21 // n) systems per
grid launch
(one system per row of the launch grid's y dimension), each with its own
vectors, state and partial sums; a system that stops ends each later launch
at its first barrier while the rest of its group goes on.  Every system of
such a batch must equal the same system solved alone, bit for bit
(solution, adjoint, gradients, iteration counts), whether its group stops
it early or late, at an even or odd iteration, at iteration 0 (zero
right-hand side, zero diagonal), with an initial guess, in fp64 and fp32,
and across several groups.  The single
solves are the ones the parity tests pin to the oracle; a few systems are
also checked against the oracle here.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import FP_TOL, banner, oracle_forward_adjoint, relerr, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _run(hip, p, x0=None):
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p),
                      build_transpose=p.method == "bicgstab")
    kw = dict(method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit, check=False)
    xin = None if x0 is None else torch.from_numpy(np.ascontiguousarray(x0)).cuda()
    x, info = pat.solve(d["val"], d["b"], x0=xin, **kw)
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **kw)
    torch.cuda.synchronize()
    out = dict(x=x.cpu().numpy(), gv=gv.cpu().numpy(), gb=gb.cpu().numpy(), info=info,
               ainfo=ainfo, ws=pat.workspace_bytes())
    pat.close()
    return out


def _one(p, s):
    return W.Problem(f"{p.name}_sys{s}", p.n, p.row_ptr, p.col, p.values[s:s + 1],
                     p.b[s:s + 1], p.x_t[s:s + 1], method=p.method, precond=p.precond,
                     tol=p.tol, maxit=p.maxit)


def _equal_to_singles(hip, p, x0=None, skip=()):
    g = _run(hip, p, x0)
    for s in range(p.batch):
        q = _one(p, s)
        gs = _run(hip, q, None if x0 is None else x0[s:s + 1])
        for key in ("status", "iters"):
            assert gs["info"][key][0] == g["info"][key][s], (p.name, s, key)
            assert gs["ainfo"][key][0] == g["ainfo"][key][s], (p.name, s, key)
        if s in skip:
            continue
        for key in ("x", "gv", "gb"):
            assert np.array_equal(gs[key][0], g[key][s]), (p.name, s, key)
    return g


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_one_group_equals_singles(hip, dtype):
    """Six 72 x 72 diffusion systems (n = 5184, one launch group), distinct
    coefficients, one zero right-hand side; with and without an initial
    guess."""
    banner(f"grid batch: one group {np.dtype(dtype).name}")
    p = W.config(3, size=72, batch=6, dtype=dtype)
    p.b[2] = 0.0
    g = _equal_to_singles(hip, p)
    its = [int(v) for v in g["info"]["iters"]]
    print("iterations per system:", its, flush=True)
    assert its[2] == 0 and not np.any(g["x"][2])
    assert len(set(its) - {0}) > 1  # the group's systems stop at different iterations
    rng = np.random.default_rng(4)
    x0 = rng.standard_normal((p.batch, p.n)).astype(dtype)
    g0 = _equal_to_singles(hip, p, x0=x0)
    assert not np.any(g0["x"][2])  # b = 0 returns x = 0 whatever the guess
    if dtype == np.float64:
        systems = [0, 5]
        r, a = oracle_forward_adjoint(p, systems=systems)
        tol = FP_TOL[np.dtype(np.float64)]["sol"]
        for j, s in enumerate(systems):
            assert relerr(g["x"][s], r.x[j]) <= tol
            assert relerr(g["gb"][s], a.grad_b[j]) <= tol
            assert relerr(g["gv"][s], a.grad_values[j]) <= tol
            assert abs(int(g["info"]["iters"][s]) - int(r.iters[j])) <= 3


def test_zero_diagonal_stops_only_its_system(hip):
    """A zero diagonal entry in one system of a Jacobi group: that system
    reports the error at iteration 0, the others solve as if alone."""
    banner("grid batch: zero diagonal in one system")
    p = W.config(3, size=72, batch=4)
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    k = int(np.flatnonzero((rows == 100) & (p.col == 100))[0])
    p.values[1, k] = 0.0
    g = _equal_to_singles(hip, p, skip=(1,))
    assert g["info"]["status"][1] == hip.SLA_ERR_ZERO_DIAG
    assert all(g["info"]["status"][s] == 0 for s in (0, 2, 3))


def test_several_groups_equal_singles(hip):
    """Three 90^3 diffusion systems (n = 729000): a group holds
    2^21 // n = 2 of them, so the batch runs as groups of 2 and 1.
    Off-diagonal entries scaled by 1, 0.9 and 0.8 (still symmetric and
    diagonally dominant) give each system its own iteration count."""
    banner("grid batch: groups of 2 + 1 at 90^3")
    q = W.config(2, size=90)
    B = 3
    rows = np.repeat(np.arange(q.n), np.diff(q.row_ptr))
    off = q.col != rows
    vals = np.repeat(q.values, B, axis=0)
    vals[:, off] *= (1.0 - 0.1 * np.arange(B))[:, None]
    rng = np.random.default_rng(12)
    p = W.Problem("diffusion90_batch3", q.n, q.row_ptr, q.col, vals,
                  rng.standard_normal((B, q.n)), rng.uniform(-1.0, 1.0, (B, q.n)),
                  method="cg", precond="jacobi", tol=1e-10, maxit=1000)
    g = _equal_to_singles(hip, p)
    its = [int(v) for v in g["info"]["iters"]]
    print("iterations per system:", its, flush=True)
    assert all(s == 0 for s in g["info"]["status"])
    assert len(set(its)) == B
    # System 1's adjoint stops (at an odd iteration) while system 0 of its
    # group runs on, so its later workgroups start around the launch that
    # stops it: a workgroup whose wavefronts disagreed on the stop flag would
    # apply one more update to some of its rows.  Repeated adjoints stay
    # bitwise equal.
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p))
    kw = dict(method="cg", precond=p.precond, tol=p.tol, maxit=p.maxit)
    x, _ = pat.solve(d["val"], d["b"], **kw)
    gx = x - d["xt"]
    for rep in range(4):
        kw["graph_chunk"] = -16 if rep % 2 else 0
        gv, gb, _ = pat.solve_adjoint(d["val"], x, gx, **kw)
        assert np.array_equal(gb.cpu().numpy(), g["gb"]), rep
        assert np.array_equal(gv.cpu().numpy(), g["gv"]), rep
    pat.close()


def _scaled_batch(q, B, seed):
    """B systems on q's pattern, system s with its off-diagonal entries
    scaled by 1 - 0.08 s (each its own iteration count), seeded right-hand
    sides and targets."""
    rows = np.repeat(np.arange(q.n), np.diff(q.row_ptr))
    off = q.col != rows
    vals = np.repeat(q.values, B, axis=0)
    vals[:, off] *= (1.0 - 0.08 * np.arange(B))[:, None]
    rng = np.random.default_rng(seed)
    return W.Problem(f"{q.name}_batch{B}", q.n, q.row_ptr, q.col, vals,
                     rng.standard_normal((B, q.n)), rng.uniform(-1.0, 1.0, (B, q.n)),
                     method=q.method, precond=q.precond, tol=q.tol, maxit=q.maxit)


def test_bicgstab_group_equals_singles(hip):
    """Four 72 x 72 upwind convection-diffusion systems (n = 5184, one
    BiCGStab launch group), one zero right-hand side; with and without an
    initial guess; two systems against the oracle."""
    banner("grid batch: BiCGStab group")
    p = _scaled_batch(W.config(4, size=72), 4, 21)
    p.b[1] = 0.0
    g = _equal_to_singles(hip, p)
    its = [int(v) for v in g["info"]["iters"]]
    print("iterations per system:", its, flush=True)
    assert its[1] == 0 and not np.any(g["x"][1])
    assert len(set(its) - {0}) > 1
    assert all(s == 0 for s in g["info"]["status"])
    rng = np.random.default_rng(5)
    _equal_to_singles(hip, p, x0=rng.standard_normal((p.batch, p.n)))
    systems = [0, 3]
    r, a = oracle_forward_adjoint(p, systems=systems)
    tol = FP_TOL[np.dtype(np.float64)]["sol"]
    for j, s in enumerate(systems):
        assert relerr(g["x"][s], r.x[j]) <= tol
        assert relerr(g["gb"][s], a.grad_b[j]) <= tol
        assert relerr(g["gv"][s], a.grad_values[j]) <= tol


def test_bicgstab_split_group_equals_singles(hip):
    """Three systems on a directed power-law graph (rows past the tile
    walker: split BiCGStab iterations, the product on the row plan) in one
    group."""
    banner("grid batch: split BiCGStab group")
    from test_gpu_row_plan import directed_graph_problem
    p = _scaled_batch(directed_graph_problem(20000, 19), 3, 22)
    g = _equal_to_singles(hip, p)
    its = [int(v) for v in g["info"]["iters"]]
    print("iterations per system:", its, flush=True)
    assert all(s == 0 for s in g["info"]["status"])
    assert len(set(its)) > 1


def test_bicgstab_several_groups_equal_singles(hip):
    """Three 800 x 800 convection-diffusion systems (n = 640000): a group
    holds 2^21 // n = 3 of them; a batch of four runs as groups of 3 and 1."""
    banner("grid batch: BiCGStab groups of 3 + 1 at 800^2")
    p = _scaled_batch(W.config(4, size=800), 4, 23)
    g = _equal_to_singles(hip, p)
    its = [int(v) for v in g["info"]["iters"]]
    print("iterations per system:", its, flush=True)
    assert all(s == 0 for s in g["info"]["status"])
    assert len(set(its)) > 1


def test_group_workspace(hip):
    """The workspace grows with the launch group only: a batch of systems
    the one-workgroup solver takes (n <= 4096) keeps one system's vectors."""
    banner("grid batch: workspace")
    small = [W.config(3, size=64, batch=b) for b in (1, 64)]
    ws = []
    for p in small:
        d = to_dev(p)
        pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p))
        ws.append(pat.workspace_bytes())
        pat.close()
    # only the per-system state (a few hundred bytes each) differs
    assert ws[1] - ws[0] < 64 * 1024, ws
    big = [W.config(3, size=72, batch=b) for b in (1, 2, 4)]
    ws = []
    for p in big:
        d = to_dev(p)
        pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p))
        ws.append(pat.workspace_bytes())
        pat.close()
    step = ws[1] - ws[0]
    assert step >= 11 * 8 * p.n  # eleven more vectors per system, at least
    assert abs((ws[2] - ws[1]) - 2 * step) <= 1024, ws
