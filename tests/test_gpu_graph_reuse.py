"""Captured iteration graphs replayed with other data.

A handle captures K iterations of a grid solve once and replays the graph in
later calls and for later launch groups of a batch.  Every pointer that can
change between calls (the caller's values, the systems' states) must reach
the kernels through the device argument blocks, never as a kernel argument
baked into the graph.  These tests keep every tensor alive (so the caching
allocator cannot hand the new tensor the old address) and check:
  - split BiCGStab (row plan) on a batch of two: each system equals its own
    single-system solve bit for bit;
  - split CG on a batch of twice the launch group: the second group replays
    the first group's graph and must still equal single-system solves;
  - one handle solving with one values tensor, then with another: the second
    solve equals a fresh handle's bit for bit and the oracle's within the
    solution bound; for the split CG and BiCGStab paths and the fused one.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import FP_TOL, banner, oracle_forward_adjoint, relerr, tdtype, to_dev
from test_gpu_row_plan import directed_graph_problem, graph_problem

pytestmark = pytest.mark.gpu

SOL = FP_TOL[np.dtype(np.float64)]["sol"]


def _run(hip, pat, d, p, **kw):
    opts = dict(method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit, check=False)
    opts.update(kw)
    x, info = pat.solve(d["val"], d["b"], **opts)
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **opts)
    torch.cuda.synchronize()
    return dict(x=x.cpu().numpy(), gv=gv.cpu().numpy(), gb=gb.cpu().numpy(), info=info,
                ainfo=ainfo)


def _single(hip, p, s):
    """System s of p solved on a fresh single-system handle."""
    q = W.Problem("one", p.n, p.row_ptr, p.col, p.values[s:s + 1], p.b[s:s + 1],
                  p.x_t[s:s + 1], method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit)
    d = to_dev(q)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(q),
                      build_transpose=(q.method == "bicgstab"))
    out = _run(hip, pat, d, q)
    pat.close()
    return out


def _batched(p, scales, seed):
    """p's single system repeated with its values scaled per system and its
    own right-hand side and target per system."""
    rng = np.random.default_rng(seed)
    B = len(scales)
    vals = np.repeat(p.values[:1], B, axis=0) * np.asarray(scales)[:, None]
    return W.Problem(p.name + f"_b{B}", p.n, p.row_ptr, p.col, vals,
                     rng.standard_normal((B, p.n)), rng.uniform(-1.0, 1.0, (B, p.n)),
                     method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit)


def _assert_same(a, b, s_a, s_b, what):
    for key in ("x", "gv", "gb"):
        assert np.array_equal(a[key][s_a], b[key][s_b]), (what, key)
    assert a["info"]["iters"][s_a] == b["info"]["iters"][s_b], what
    assert a["ainfo"]["iters"][s_a] == b["ainfo"]["iters"][s_b], what


def test_split_bicgstab_batch_of_two(hip):
    """One system per launch group: the second group replays the first's
    graph with its own values and state."""
    banner("graph reuse: split bicgstab batch 2")
    p = _batched(directed_graph_problem(20000, 19), [1.0, 1.25], 31)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=2, dtype=tdtype(p), build_transpose=True)
    assert pat.iteration_form() != "diagonal-major"  # the row plan's split path
    g = _run(hip, pat, d, p)
    for s in range(2):
        assert g["info"]["status"][s] == 0 and g["ainfo"]["status"][s] == 0, s
        _assert_same(g, _single(hip, p, s), s, 0, f"system {s}")
    r, a = oracle_forward_adjoint(p, systems=[1])
    assert relerr(g["x"][1], r.x[0]) <= SOL
    assert relerr(g["gb"][1], a.grad_b[0]) <= SOL
    pat.close()


def test_split_cg_two_launch_groups(hip):
    """n = 700 000 rows: two systems per launch group, so a batch of four
    runs two groups with the same captured graph."""
    banner("graph reuse: split cg, batch of two launch groups")
    p = graph_problem(700000, 23, batch=4)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=4, dtype=tdtype(p))
    # a launch group holds min(batch, 2^21 // n) systems of more than 4096 rows
    assert (1 << 21) // p.n == 2
    g = _run(hip, pat, d, p)
    pat.close()
    for s in range(4):
        assert g["info"]["status"][s] == 0 and g["ainfo"]["status"][s] == 0, s
        _assert_same(g, _single(hip, p, s), s, 0, f"system {s}")
    r, a = oracle_forward_adjoint(p, systems=[3])
    assert relerr(g["x"][3], r.x[0]) <= SOL
    assert relerr(g["gv"][3], a.grad_values[0]) <= SOL


def _second_values(p, seed):
    """p with each stored value scaled by its own factor in [0.8, 1.2],
    symmetric pairs scaled alike (so CG still sees a symmetric matrix) and
    the diagonal reset to dominate its row."""
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    lo = np.minimum(rows, p.col).astype(np.int64)
    hi = np.maximum(rows, p.col).astype(np.int64)
    h = (lo * 1000003 + hi * 7919 + seed) % 4001
    v = p.values[0] * (0.8 + 0.4 * h / 4000.0)
    off = rows != p.col
    dsum = np.zeros(p.n)
    np.add.at(dsum, rows[off], np.abs(v[off]))
    v = v.copy()
    v[~off] = dsum[rows[~off]] + 1.0
    return W.Problem(p.name + "_v2", p.n, p.row_ptr, p.col, v[None, :], p.b, p.x_t,
                     method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit)


CASES = {
    "split_cg": lambda: graph_problem(30000, 13),
    "split_bicgstab": lambda: directed_graph_problem(20000, 19),
    "fused_cg_3d": lambda: W.config(2, size=24),
}


@pytest.mark.parametrize("case", list(CASES))
def test_new_values_on_one_handle(hip, case):
    banner(f"graph reuse: new values on one handle ({case})")
    p1 = CASES[case]()
    p2 = _second_values(p1, 5)
    d1, d2 = to_dev(p1), to_dev(p2)
    bt = p1.method == "bicgstab"
    pat = hip.Pattern(d1["rp"], d1["col"], dtype=tdtype(p1), build_transpose=bt)
    g1 = _run(hip, pat, d1, p1)
    g2 = _run(hip, pat, d2, p2)  # d1 stays alive: a new address for the values
    assert d1["val"].data_ptr() != d2["val"].data_ptr()
    fresh = _single(hip, p2, 0)
    _assert_same(g2, fresh, 0, 0, "second values")
    r, a = oracle_forward_adjoint(p2)
    assert g2["info"]["status"][0] == 0 and g2["ainfo"]["status"][0] == 0
    assert relerr(g2["x"][0], r.x[0]) <= SOL
    assert relerr(g2["gb"][0], a.grad_b[0]) <= SOL
    assert relerr(g2["gv"][0], a.grad_values[0]) <= SOL
    # and back to the first tensor: the first solve again, bit for bit
    g3 = _run(hip, pat, d1, p1)
    _assert_same(g3, g1, 0, 0, "first values again")
    pat.close()
