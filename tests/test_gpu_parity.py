"""GPU parity: the HIP path (through the C ABI) against the oracle on the same
seeded inputs.

Bars (fp64 / fp32): SpMV componentwise |dy_i| <= tol * sum_j |A_ij||x_j| with
tol 1e-12 / 1e-5; converged solves and gradients relative L2 <= 1e-7 / 1e-3
when both sides reach ||r||/||b|| <= tol.  Integer set-up outputs (diagonal
index, transpose map) are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import (FP_TOL, banner, gpu_forward_adjoint, oracle_forward_adjoint, relerr,
                         spmv_bound, tdtype, to_dev)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ set-up

# The transpose map comes from a radix sort of (column, entry) pairs, eight
# bits per pass: n = 36 takes one pass, 300 / 4096 / 5000 / 64 000 two,
# 2^18 three.  Columns of a tile of 4096 entries spread over many digits
# (random, power-law) or few (stencils).
def _random_pattern(n, k, seed):
    """Each row: its diagonal and k columns drawn uniformly (repeats merged)."""
    rng = np.random.default_rng(seed)
    c = np.concatenate([rng.integers(0, n, size=(n, k)), np.arange(n)[:, None]], axis=1)
    c.sort(axis=1)
    keep = np.ones(c.shape, dtype=bool)
    keep[:, 1:] = c[:, 1:] != c[:, :-1]
    rp = np.zeros(n + 1, dtype=np.int32)
    rp[1:] = np.cumsum(keep.sum(axis=1))
    return rp, c[keep].astype(np.int32)


SETUP_CASES = ["laplace_6", "convdiff_64", "random_nonsym_300", "powerlaw_5000", "poisson_i64",
               "diffusion3d_40", "random_nonsym_70000", "powerlaw_2^18"]


@pytest.mark.parametrize("case", SETUP_CASES)
def test_pattern_setup_bit_exact(hip, case):
    banner(f"setup {case}")
    if case == "laplace_6":
        rp, col, _ = W.laplacian_2d(6)
    elif case == "convdiff_64":
        p = W.config(4, size=64)
        rp, col = p.row_ptr, p.col
    elif case == "random_nonsym_300":
        rp, col, _ = W.random_csr(300, 0.05, 3)
    elif case == "random_nonsym_70000":
        rp, col = _random_pattern(70000, 6, 5)
    elif case == "powerlaw_5000":
        rp, col, _ = W.powerlaw_graph_laplacian(5000, 4)
    elif case == "powerlaw_2^18":
        rp, col, _ = W.powerlaw_graph_laplacian(1 << 18, 6)
    elif case == "diffusion3d_40":
        p = W.config(2, size=40)
        rp, col = p.row_ptr, p.col
    else:
        p = W.config(5, size=9)
        rp, col = p.row_ptr, p.col
    n = rp.shape[0] - 1
    st, dp = O.check_pattern(n, rp, col)
    assert st == O.OK
    rpt, ct, perm = O.transpose(n, rp, col)
    drp = torch.from_numpy(rp).cuda()
    dcol = torch.from_numpy(col).cuda()
    pat = hip.Pattern(drp, dcol, batch=1, dtype=torch.float64, build_transpose=True)
    g_dp, g_rpt, g_ct, g_perm = pat.export_pattern()
    torch.cuda.synchronize()
    assert np.array_equal(g_dp.cpu().numpy().astype(np.int64), dp)
    assert np.array_equal(g_rpt.cpu().numpy().astype(np.int64), rpt)
    assert np.array_equal(g_ct.cpu().numpy(), ct)
    assert np.array_equal(g_perm.cpu().numpy().astype(np.int64), perm)


def test_invalid_patterns_rejected(hip):
    banner("invalid patterns")
    rp, col, _ = W.laplacian_2d(6)
    n = 36
    cases = []
    bad = col.copy(); bad[1], bad[2] = bad[2], bad[1]; cases.append((rp, bad))
    bad = col.copy(); bad[-1] = n; cases.append((rp, bad))
    bad = col.copy(); bad[1] = bad[0]; cases.append((rp, bad))
    rp2 = rp.copy(); rp2[5] = rp2[6] + 1; cases.append((rp2, col))
    rp3 = rp.copy(); rp3[0] = 1; cases.append((rp3, col))
    cases.append((np.array([0, 1, 2], dtype=np.int32), np.array([1, 0], dtype=np.int32)))
    for r, c in cases:
        assert O.check_pattern(r.shape[0] - 1, r, c)[0] == O.ERR_PATTERN
        with pytest.raises(hip.SlaError) as ei:
            hip.Pattern(torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda())
        assert ei.value.status == hip.SLA_ERR_PATTERN


# ------------------------------------------------------------------ SpMV

def _spmv_case(hip, p, transpose=False):
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p), build_transpose=transpose)
    rng = np.random.default_rng(17)
    x = rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)
    y = pat.matvec(d["val"], torch.from_numpy(x).cuda(), transpose=transpose).cpu().numpy()
    tol = FP_TOL[p.values.dtype]["spmv"]
    if transpose:
        rpt, ct, perm = O.transpose(p.n, p.row_ptr, p.col)
    for s in range(p.batch):
        if transpose:
            vt = p.values[s].astype(np.float64)[perm]
            ref = O.spmv(rpt, ct, vt, x[s].astype(np.float64))
            bound = tol * O.spmv(rpt, ct, np.abs(vt), np.abs(x[s].astype(np.float64))) + 1e-300
        else:
            ref = O.spmv(p.row_ptr, p.col, p.values[s].astype(np.float64), x[s].astype(np.float64))
            bound = spmv_bound(p, x[s], s, tol)
        err = np.abs(y[s].astype(np.float64) - ref)
        assert np.all(err <= bound), f"{p.name} sys {s}: worst {np.max(err / bound)}"


@pytest.mark.parametrize("k", [1, 2, 4])
def test_spmv_full_configs(hip, k):
    banner(f"spmv config {k}")
    _spmv_case(hip, W.config(k), transpose=(k == 4))


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_spmv_batched_shared_pattern(hip, dtype):
    banner(f"spmv batched {np.dtype(dtype).name}")
    _spmv_case(hip, W.config(3, dtype=dtype))


@pytest.mark.parametrize("size", [1, 3, 7, 17])
def test_spmv_ragged_and_tiny(hip, size):
    banner(f"spmv ragged {size}")
    _spmv_case(hip, W.config(2, size=size), transpose=True)


def test_spmv_long_rows_powerlaw(hip):
    banner("spmv powerlaw")
    rp, col, val = W.powerlaw_graph_laplacian(60000, 9)
    p = W.Problem("powerlaw", 60000, rp, col, val, np.zeros((1, 60000)), np.zeros((1, 60000)))
    _spmv_case(hip, p, transpose=True)


def test_spmv_int64_row_ptr(hip):
    banner("spmv int64")
    p = W.config(5, size=40)
    _spmv_case(hip, p)


# ------------------------------------------------------------------ product backward

def _vjp_case(hip, p):
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p), build_transpose=True)
    rng = np.random.default_rng(23)
    x = rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)
    g = rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)
    gv, gx = pat.matvec_adjoint(d["val"], torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda())
    gv, gx = gv.cpu().numpy(), gx.cpu().numpy()
    tol = FP_TOL[p.values.dtype]["spmv"]
    rpt, ct, perm = O.transpose(p.n, p.row_ptr, p.col)
    for s in range(p.batch):
        v = p.values[s].astype(np.float64)
        ogx, ogv = O.matvec_vjp(p.row_ptr, p.col, v, x[s].astype(np.float64),
                                g[s].astype(np.float64))
        bound = tol * O.spmv(rpt, ct, np.abs(v[perm]), np.abs(g[s].astype(np.float64))) + 1e-300
        err = np.abs(gx[s].astype(np.float64) - ogx)
        assert np.all(err <= bound), f"{p.name} sys {s}: grad_x worst {np.max(err / bound)}"
        # one product per entry: the GPU's rounding of g_i x_j is the exact
        # product rounded to the working precision, as is the oracle's
        assert np.array_equal(gv[s], ogv.astype(p.values.dtype)), f"{p.name} sys {s}: grad_values"


@pytest.mark.parametrize("case", ["convdiff_40", "random_nonsym_300", "batched_fp64",
                                  "batched_fp32", "powerlaw", "cfg2_full"])
def test_matvec_adjoint_matches_oracle(hip, case):
    banner(f"matvec adjoint {case}")
    if case == "convdiff_40":
        p = W.config(4, size=40)
    elif case == "random_nonsym_300":
        rp, col, val = W.random_csr(300, 0.05, 3)
        p = W.Problem("random300", 300, rp, col, val, np.zeros((1, 300)), np.zeros((1, 300)))
    elif case == "batched_fp64":
        p = W.config(3, size=20, batch=5)
    elif case == "batched_fp32":
        p = W.config(3, size=20, batch=5, dtype=np.float32)
    elif case == "powerlaw":
        rp, col, val = W.powerlaw_graph_laplacian(60000, 9)
        p = W.Problem("powerlaw", 60000, rp, col, val, np.zeros((1, 60000)), np.zeros((1, 60000)))
    else:
        p = W.config(2)
    _vjp_case(hip, p)


def test_matvec_adjoint_arguments(hip):
    banner("matvec adjoint arguments")
    p = W.config(4, size=16)
    d = to_dev(p)
    x = torch.randn(p.n, dtype=torch.float64, device="cuda")
    pat = hip.Pattern(d["rp"], d["col"])  # no transpose map
    with pytest.raises(hip.SlaError) as ei:
        pat.matvec_adjoint(d["val"], x, x)
    assert ei.value.status == hip.SLA_ERR_ARG
    gv, gx = pat.matvec_adjoint(d["val"], x, x, need_grad_x=False)  # values only: no map needed
    assert gx is None and gv.shape == d["val"].shape
    with pytest.raises(hip.SlaError):
        pat.matvec_adjoint(d["val"], x, x, need_grad_x=False, need_grad_values=False)


@pytest.mark.parametrize("case", ["cfg2_30", "cfg4_40", "cfg3_batch3_fp32"])
def test_matvec_adjoint_outputs_alone_equal_both(hip, case):
    """With diagonal masks one kernel makes grad_x and grad_values together;
    asking for either alone gives bitwise the same arrays."""
    banner(f"matvec adjoint alone vs both {case}")
    p = {"cfg2_30": lambda: W.config(2, size=30), "cfg4_40": lambda: W.config(4, size=40),
         "cfg3_batch3_fp32": lambda: W.config(3, size=24, batch=3, dtype=np.float32)}[case]()
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p), build_transpose=True)
    assert pat.column_mode() == "diagonal"
    rng = np.random.default_rng(31)
    x = torch.from_numpy(rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)).cuda()
    g = torch.from_numpy(rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)).cuda()
    gv, gx = pat.matvec_adjoint(d["val"], x, g)
    gv1, _ = pat.matvec_adjoint(d["val"], x, g, need_grad_x=False)
    _, gx1 = pat.matvec_adjoint(d["val"], x, g, need_grad_values=False)
    yt = pat.matvec(d["val"], g, transpose=True)
    assert torch.equal(gv, gv1) and torch.equal(gx, gx1) and torch.equal(gx, yt)


def test_sparse_matvec_autograd(hip):
    banner("autograd matvec")
    rp, col, val = W.random_csr(50, 0.2, 9, symmetric=False)
    rows = torch.from_numpy(np.repeat(np.arange(50), np.diff(rp)))
    cols = torch.from_numpy(col.astype(np.int64))
    pat = hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda(),
                      build_transpose=True)
    v = torch.from_numpy(val[0].copy()).cuda().requires_grad_(True)
    x = torch.randn(50, dtype=torch.float64, device="cuda", requires_grad=True)
    w = torch.randn(50, dtype=torch.float64, device="cuda")
    loss = (hip.sparse_matvec(pat, v, x) * w).sum()
    loss.backward()
    # the same loss through a dense CPU matrix
    vc = v.detach().cpu().requires_grad_(True)
    xc = x.detach().cpu().requires_grad_(True)
    A = torch.zeros(50, 50, dtype=torch.float64).index_put((rows, cols), vc)
    lc = ((A @ xc) * w.cpu()).sum()
    lc.backward()
    assert torch.allclose(v.grad.cpu(), vc.grad, rtol=1e-14, atol=1e-14)
    assert torch.allclose(x.grad.cpu(), xc.grad, rtol=1e-12, atol=1e-13)
    assert abs(loss.item() - lc.item()) <= 1e-12 * abs(lc.item())


def test_pattern_list_is_a_loop_of_patterns(hip):
    banner("pattern list")
    probs = [W.config(1), W.config(4, size=24), W.config(2, size=9)]
    devs = [to_dev(p) for p in probs]
    plist = hip.PatternList([(d["rp"], d["col"]) for d in devs], build_transpose=True)
    assert len(plist) == 3
    xs = [torch.randn(p.n, dtype=torch.float64, device="cuda") for p in probs]
    ys = plist.matvec([d["val"] for d in devs], xs)
    outs = plist.solve([d["val"] for d in devs], [d["b"] for d in devs], tol=1e-10, maxit=4000,
                       method="bicgstab", precond="none")
    for p, d, x, y, (xsol, info) in zip(probs, devs, xs, ys, outs):
        single = hip.Pattern(d["rp"], d["col"], build_transpose=True)
        assert torch.equal(y, single.matvec(d["val"], x))
        xs1, info1 = single.solve(d["val"], d["b"], tol=1e-10, maxit=4000, method="bicgstab",
                                  precond="none")
        assert torch.equal(xsol, xs1) and info["iters"][0] == info1["iters"][0]
        r = O.solve(p.row_ptr, p.col, p.values, p.b, "bicgstab", "none", 1e-10, 4000)
        assert relerr(xsol.cpu().numpy()[0], r.x[0]) <= 1e-7


# ------------------------------------------------------------------ solves

def _check_solve(p, g, r, a, systems=None):
    systems = list(range(p.batch)) if systems is None else list(systems)
    tol = FP_TOL[p.values.dtype]["sol"]
    for j, s in enumerate(systems):
        assert g["info"]["status"][s] == 0 and r.status[j] == 0, (p.name, s)
        assert g["ainfo"]["status"][s] == 0 and a.status[j] == 0, (p.name, s)
        ex = relerr(g["x"][s], r.x[j])
        egv = relerr(g["gv"][s], a.grad_values[j])
        egb = relerr(g["gb"][s], a.grad_b[j])
        assert ex <= tol and egv <= tol and egb <= tol, (p.name, s, ex, egv, egb)
        # iteration counts agree up to reduction-order effects
        assert abs(int(g["info"]["iters"][s]) - int(r.iters[j])) <= max(3, r.iters[j] // 50)


@pytest.mark.parametrize("case", ["cfg1", "cfg1_grid", "cfg2_20", "cfg2_31_ragged", "cfg3_small64",
                                  "cfg3_small32", "cfg4_48", "cfg4_33_ragged", "cfg2_24_fp32",
                                  "cfg4_40_fp32", "cfg5_20_fp32", "cfg4_40_i64"])
def test_solve_and_adjoint_small(hip, case):
    banner(f"solve {case}")
    kw = {}
    if case == "cfg1":
        p = W.config(1)
    elif case == "cfg1_grid":
        p = W.config(1)
        kw["profile"] = True   # forces the grid kernels on a small system
    elif case == "cfg2_20":
        p = W.config(2, size=20)
    elif case == "cfg2_24_fp32":
        # fp32 on the grid kernels (n = 13 824): tol 1e-5, fp64 dot products
        p = W.config(2, size=24).astype(np.float32)
        p.tol = 1e-5
    elif case == "cfg4_40_fp32":
        p = W.config(4, size=40).astype(np.float32)
        p.tol = 1e-5
    elif case == "cfg5_20_fp32":
        # int64 row_ptr with fp32 values on the grid kernels (n = 8000)
        p = W.config(5, size=20).astype(np.float32)
        p.tol = 1e-5
    elif case == "cfg4_40_i64":
        # BiCGStab and its transpose map with an int64 row_ptr
        p = W.config(4, size=40)
        p.row_ptr = p.row_ptr.astype(np.int64)
    elif case == "cfg2_31_ragged":
        p = W.config(2, size=31)
    elif case == "cfg3_small64":
        p = W.config(3, size=20, batch=16)
    elif case == "cfg3_small32":
        p = W.config(3, size=20, batch=16, dtype=np.float32)
    elif case == "cfg4_48":
        p = W.config(4, size=48)
    else:
        p = W.config(4, size=33)
    g = gpu_forward_adjoint(hip, p, **kw)
    r, a = oracle_forward_adjoint(p)
    _check_solve(p, g, r, a)


def test_solve_config2_full(hip):
    banner("solve config 2 full")
    p = W.config(2)
    g = gpu_forward_adjoint(hip, p)
    r, a = oracle_forward_adjoint(p)
    _check_solve(p, g, r, a)
    tr = O.true_relres(p.row_ptr, p.col, p.values, g["x"], p.b)
    assert tr[0] <= 10 * p.tol


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_solve_config3_full_batch(hip, dtype):
    banner(f"solve config 3 full {np.dtype(dtype).name}")
    p = W.config(3, dtype=dtype)
    g = gpu_forward_adjoint(hip, p)
    sample = list(range(0, p.batch, 32)) + [p.batch - 1]
    r, a = oracle_forward_adjoint(p, systems=sample)
    gs = dict(g)
    _check_solve(p, gs, r, a, systems=sample)
    # every system: converged, and the oracle's true residual confirms it
    assert np.all(g["info"]["status"] == 0) and np.all(g["ainfo"]["status"] == 0)
    tr = O.true_relres(p.row_ptr, p.col, p.values.astype(np.float64), g["x"].astype(np.float64),
                       p.b.astype(np.float64))
    limit = 10 * p.tol if dtype == np.float64 else 1e-3
    assert np.all(tr <= limit), float(tr.max())


def test_solve_config4_full(hip):
    banner("solve config 4 full")
    p = W.config(4)
    g = gpu_forward_adjoint(hip, p)
    r, a = oracle_forward_adjoint(p)
    _check_solve(p, g, r, a)
    assert g["info"]["iters"][0] < p.maxit


# ------------------------------------------------------------------ edge cases

def test_fixed_iteration_count_matches_oracle_iterates(hip):
    banner("fixed iterations")
    for p, path in ((W.config(2, size=24), {}), (W.config(1), {}), (W.config(1), {"profile": True}),
                    (W.config(4, size=40), {})):
        for k in (1, 2, 7):
            g = gpu_forward_adjoint(hip, p, maxit=k, **path)
            r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, p.tol, k)
            assert g["info"]["status"][0] == hip.SLA_NOT_CONVERGED, (p.name, k, path, g["info"])
            assert r.status[0] == O.NOT_CONVERGED
            assert g["info"]["iters"][0] == k == r.iters[0]
            assert relerr(g["x"][0], r.x[0]) <= 1e-12, (p.name, k, path)
            assert abs(g["info"]["relres"][0] - r.relres[0]) <= 1e-10 * r.relres[0]


def test_zero_rhs_and_zero_maxit(hip):
    banner("zero rhs / maxit 0")
    for p in (W.config(1), W.config(2, size=12), W.config(4, size=16)):
        d = to_dev(p)
        pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
        for kw in ({}, {"profile": True}):
            x, info = pat.solve(d["val"], torch.zeros_like(d["b"]), method=p.method,
                                precond=p.precond, **kw)
            assert info["status"][0] == 0 and info["iters"][0] == 0
            assert not torch.any(x)
            x0 = torch.ones_like(d["b"])
            x, info = pat.solve(d["val"], torch.zeros_like(d["b"]), method=p.method,
                                precond=p.precond, x0=x0, **kw)
            assert info["status"][0] == 0 and not torch.any(x)
            x, info = pat.solve(d["val"], d["b"], maxit=0, method=p.method, precond=p.precond,
                                check=False, **kw)
            assert info["return"] == hip.SLA_NOT_CONVERGED and info["iters"][0] == 0
            assert not torch.any(x)


def test_initial_guess(hip):
    banner("initial guess")
    # (config 2 at 16^3 and config 1 run on the one-workgroup solver, config 2
    # at 20^3 on the grid kernels with the diagonal-major values)
    for p, kw in ((W.config(2, size=16), {}), (W.config(2, size=20), {}), (W.config(1), {}),
                  (W.config(4, size=24), {})):
        d = to_dev(p)
        pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
        x, info = pat.solve(d["val"], d["b"], tol=1e-12, maxit=5000, method=p.method,
                            precond=p.precond)
        x2, info2 = pat.solve(d["val"], d["b"], tol=1e-10, maxit=5000, method=p.method,
                              precond=p.precond, x0=x)
        assert info2["status"][0] == 0 and info2["iters"][0] == 0
        rng = np.random.default_rng(3)
        x0 = torch.from_numpy(rng.standard_normal((1, p.n))).cuda()
        x3, info3 = pat.solve(d["val"], d["b"], tol=1e-11, maxit=5000, method=p.method,
                              precond=p.precond, x0=x0)
        assert info3["status"][0] == 0
        assert relerr(x3.cpu().numpy(), x.cpu().numpy()) <= 1e-7


def test_zero_diagonal_and_breakdown(hip):
    banner("zero diag / breakdown")
    p = W.config(1, size=8)
    st, dp = O.check_pattern(p.n, p.row_ptr, p.col)
    v = p.values.copy()
    v[0, dp[5]] = 0.0
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=torch.float64)
    for kw in ({}, {"profile": True}):
        with pytest.raises(hip.SlaError) as ei:
            pat.solve(torch.from_numpy(v).cuda(), d["b"], precond="jacobi", **kw)
        assert ei.value.status == hip.SLA_ERR_ZERO_DIAG
    # indefinite symmetric diagonal: p.Ap <= 0
    rp = torch.tensor([0, 1, 2], dtype=torch.int32).cuda()
    col = torch.tensor([0, 1], dtype=torch.int32).cuda()
    pat2 = hip.Pattern(rp, col, dtype=torch.float64, build_transpose=True)
    vals = torch.tensor([[1.0, -1.0]], dtype=torch.float64).cuda()
    bb = torch.tensor([[0.0, 1.0]], dtype=torch.float64).cuda()
    for kw in ({}, {"profile": True}):
        x, info = pat2.solve(vals, bb, precond="none", check=False, **kw)
        assert info["return"] == hip.SLA_BREAKDOWN
    # BiCGStab: rhat.v = 0 for A = [[0,1],[1,0]], b = e1
    rp = torch.tensor([0, 2, 4], dtype=torch.int32).cuda()
    col = torch.tensor([0, 1, 0, 1], dtype=torch.int32).cuda()
    pat3 = hip.Pattern(rp, col, dtype=torch.float64, build_transpose=True)
    vals = torch.tensor([[0.0, 1.0, 1.0, 0.0]], dtype=torch.float64).cuda()
    bb = torch.tensor([[1.0, 0.0]], dtype=torch.float64).cuda()
    x, info = pat3.solve(vals, bb, method="bicgstab", precond="none", check=False)
    assert info["return"] == hip.SLA_BREAKDOWN


def test_bicgstab_half_step(hip):
    banner("bicgstab half step")
    N = 32
    rp, col, val = W.laplacian_2d(N)
    pp = np.arange(1, N + 1)
    h = np.pi / (N + 1)
    v = np.outer(np.sin(9 * pp * h), np.sin(5 * pp * h)).reshape(-1)
    lam = 4 - 2 * np.cos(5 * h) - 2 * np.cos(9 * h)
    pat = hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda(),
                      build_transpose=True)
    x, info = pat.solve(torch.from_numpy(val).cuda(), torch.from_numpy(v[None, :]).cuda(),
                        method="bicgstab", precond="none")
    assert info["iters"][0] == 1 and info["spmv"][0] == 1
    assert relerr(x.cpu().numpy()[0], v / lam) <= 1e-13


def test_single_unknown(hip):
    banner("n = 1")
    rp = torch.tensor([0, 1], dtype=torch.int32).cuda()
    col = torch.tensor([0], dtype=torch.int32).cuda()
    pat = hip.Pattern(rp, col, dtype=torch.float64, build_transpose=True)
    vals = torch.tensor([[4.0]], dtype=torch.float64).cuda()
    b = torch.tensor([[2.0]], dtype=torch.float64).cuda()
    for m, pre in (("cg", "jacobi"), ("cg", "none"), ("bicgstab", "none")):
        x, info = pat.solve(vals, b, method=m, precond=pre)
        assert abs(x.item() - 0.5) <= 1e-15
        gv, gb, _ = pat.solve_adjoint(vals, x, x - 1.0, method=m, precond=pre)
        assert abs(gb.item() - (-0.5 / 4.0)) <= 1e-15
        assert abs(gv.item() - (0.5 / 4.0) * 0.5) <= 1e-15


def test_batch_mixed_convergence_is_loop_of_singles(hip):
    banner("batch = loop")
    p = W.config(3, size=24, batch=6)
    p.b[2] = 0.0
    g = gpu_forward_adjoint(hip, p)
    for s in range(p.batch):
        q = W.Problem("one", p.n, p.row_ptr, p.col, p.values[s:s + 1], p.b[s:s + 1],
                      p.x_t[s:s + 1], method="cg", precond="jacobi", tol=p.tol, maxit=p.maxit)
        gs = gpu_forward_adjoint(hip, q)
        assert np.array_equal(gs["x"][0], g["x"][s])
        assert gs["info"]["iters"][0] == g["info"]["iters"][s]
    assert g["info"]["iters"][2] == 0 and not np.any(g["x"][2])


def test_grid_path_batch_is_loop_of_singles(hip):
    """Batched systems on the grid kernels (n > 4096): CG advances the batch
    in one launch group, BiCGStab runs the systems one after another through
    the same graphs, diagonal-major buffer and transposed values; each
    system's results equal a single-system solve bit for bit and match the
    oracle, and a zero right-hand side inside the batch stops at 0."""
    banner("grid batch = loop")
    p3 = W.config(3, size=72, batch=3)  # CG + Jacobi, n = 5184
    p3.b[1] = 0.0
    p4 = W.config(4, size=72)  # BiCGStab
    B = 3
    rows = np.repeat(np.arange(p4.n), np.diff(p4.row_ptr))
    off = p4.col != rows
    vals = np.repeat(p4.values, B, axis=0)
    vals[:, off] *= (1.0 - 0.1 * np.arange(B))[:, None]  # stays diagonally dominant
    rng = np.random.default_rng(9)
    p4b = W.Problem("convdiff72_batch3", p4.n, p4.row_ptr, p4.col, vals,
                    rng.standard_normal((B, p4.n)), rng.uniform(-1.0, 1.0, (B, p4.n)),
                    method="bicgstab", precond="none", tol=1e-10, maxit=2000)
    for p in (p3, p4b):
        g = gpu_forward_adjoint(hip, p)
        assert g["pattern"].iteration_form() == "diagonal-major", p.name
        for s in range(p.batch):
            q = W.Problem("one", p.n, p.row_ptr, p.col, p.values[s:s + 1], p.b[s:s + 1],
                          p.x_t[s:s + 1], method=p.method, precond=p.precond, tol=p.tol,
                          maxit=p.maxit)
            gs = gpu_forward_adjoint(hip, q)
            for key in ("x", "gv", "gb"):
                assert np.array_equal(gs[key][0], g[key][s]), (p.name, s, key)
            assert gs["info"]["iters"][0] == g["info"]["iters"][s]
            assert gs["ainfo"]["iters"][0] == g["ainfo"]["iters"][s]
        systems = [s for s in range(p.batch) if np.any(p.b[s])]
        r, a = oracle_forward_adjoint(p, systems=systems)
        _check_solve(p, g, r, a, systems=systems)
        if p is p3:
            assert g["info"]["iters"][1] == 0 and not np.any(g["x"][1])


def test_determinism_and_launch_modes_agree(hip):
    banner("determinism")
    for p in (W.config(2, size=28), W.config(4, size=40)):
        d = to_dev(p)
        pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
        outs = []
        for kw in ({}, {}, {"graph_chunk": -8}, {"graph_chunk": 3}, {"profile": True}):
            x, info = pat.solve(d["val"], d["b"], method=p.method, precond=p.precond, **kw)
            gv, gb, _ = pat.solve_adjoint(d["val"], x, x - d["xt"], method=p.method,
                                          precond=p.precond, **kw)
            outs.append((x.cpu().numpy(), gv.cpu().numpy(), gb.cpu().numpy(), info["iters"][0]))
        for o in outs[1:]:
            assert all(np.array_equal(a, b) for a, b in zip(o[:3], outs[0][:3]))
            assert o[3] == outs[0][3]


def test_replay_length_changes_nothing(hip):
    """The default chunk length follows the handle's previous grid solve:
    16 iterations on a fresh handle, 32 once a solve of the 1e6-DOF workload
    has taken its ~480 iterations (at this size the chunks are launched
    directly).  Those, and graph replays of 64 and 2 iterations, give
    bitwise the same solutions, adjoints and iteration counts."""
    banner("replay lengths, 1e6 DOF")
    p = W.config(2)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p))
    outs = []
    for kw in ({}, {}, {"graph_chunk": 64}, {"graph_chunk": 2}):
        x, info = pat.solve(d["val"], d["b"], method=p.method, precond=p.precond, tol=p.tol,
                            maxit=p.maxit, **kw)
        gv, gb, ai = pat.solve_adjoint(d["val"], x, x - d["xt"], method=p.method,
                                       precond=p.precond, tol=p.tol, maxit=p.maxit, **kw)
        outs.append((x.cpu().numpy(), gv.cpu().numpy(), gb.cpu().numpy(),
                     int(info["iters"][0]), int(ai["iters"][0])))
    assert outs[0][3] >= 460 and outs[0][4] >= 460  # later solves replay 32 at a time
    for o in outs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(o[:3], outs[0][:3]))
        assert o[3:] == outs[0][3:]
    pat.close()


def test_compact_columns_change_nothing(hip):
    """The compact column forms (2-byte tile-relative columns, per-row
    diagonal masks) and the diagonal-major values of the solver iterations
    are storage choices: products, solves and adjoints are bitwise the same
    as with the caller's int32 columns and CSR values, and each form is kept
    only where it fits."""
    banner("compact columns")
    rp, col, val = W.random_csr(300, 0.05, 3)
    rnd = W.Problem("random300", 300, rp, col, val, np.ones((1, 300)), np.zeros((1, 300)),
                    method="bicgstab", precond="none", tol=1e-10, maxit=2000)
    # (problem, product form, iteration form with diagonal-major allowed)
    cases = [(W.config(2, size=28), "diagonal", "diagonal-major"),
             (W.config(4, size=40), "diagonal", "diagonal-major"),
             (W.config(3, size=20, batch=4), "diagonal", "diagonal-major"),
             (W.config(5, size=33), "diagonal", "diagonal-major"),
             (W.config(1), "diagonal", "diagonal-major"),
             (rnd, "tile16", "tile16")]
    variants = [(True, True), (True, False), (False, True)]  # (compact, diagonal-major)
    for p, mode, form in cases:
        d = to_dev(p)
        outs, ws = [], []
        for compact, dmaj in variants:
            pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p),
                              build_transpose=True, compact_columns=compact,
                              diagonal_major=dmaj)
            want = mode if compact else "wide"
            assert pat.column_mode() == want, p.name
            assert pat.column_mode(transpose=True) == want, p.name
            want_it = form if (compact and dmaj) else want
            assert pat.iteration_form() == want_it, p.name
            assert pat.iteration_form(transpose=True) == want_it, p.name
            ws.append(pat.workspace_bytes())
            xr = torch.from_numpy(np.random.default_rng(5).standard_normal((p.batch, p.n))
                                  .astype(p.values.dtype)).cuda()
            y = pat.matvec(d["val"], xr)
            yt = pat.matvec(d["val"], xr, transpose=True)
            res = [y, yt]
            for prof in (False, True):  # profile mode: the grid path at every size
                kw = dict(method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit,
                          profile=prof)
                x, info = pat.solve(d["val"], d["b"], **kw)
                gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **kw)
                res += [x, gv, gb, torch.from_numpy(np.asarray(info["iters"])),
                        torch.from_numpy(np.asarray(ainfo["iters"]))]
            outs.append([t.cpu().numpy() for t in res])
            pat.close()
        for o in outs[1:]:
            for a, b in zip(outs[0], o):
                assert np.array_equal(a, b), p.name
        # with per-entry columns (the wide form, and tile16) the handle also
        # keeps the two-pass A^T products' write positions, 6 bytes per entry,
        # which the diagonal-mask form does not need
        extra = 6 * p.nnz if mode == "diagonal" else 0
        assert ws[1] > ws[2] - extra, (p.name, ws)
        assert (ws[0] > ws[1]) == (form == "diagonal-major"), (p.name, ws)
    # offsets beyond int16 and more than 16 diagonals: no compact form
    rp, col, val = W.powerlaw_graph_laplacian(60000, 9)
    drp, dcol = torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda()
    a = hip.Pattern(drp, dcol, compact_columns=True)
    b = hip.Pattern(drp, dcol, compact_columns=False)
    assert a.column_mode() == "wide" and a.workspace_bytes() == b.workspace_bytes()


def test_workspace_independent_of_iterations(hip):
    banner("memory vs maxit")
    p = W.config(2, size=24)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p))
    ws0 = pat.workspace_bytes()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for maxit in (10, 1000):
        x, info = pat.solve(d["val"], d["b"], maxit=maxit, check=False)
        pat.solve_adjoint(d["val"], x, x - d["xt"], maxit=maxit, check=False)
        torch.cuda.synchronize()
        assert pat.workspace_bytes() == ws0
    assert torch.cuda.mem_get_info()[0] >= free0 - (64 << 20)
    assert ws0 < 40 * 8 * p.n + 4 * (1 << 20)


def test_autograd_function(hip):
    banner("autograd")
    p = W.config(4, size=20)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=torch.float64, build_transpose=True)
    vals = d["val"].clone().requires_grad_(True)
    b = d["b"].clone().requires_grad_(True)
    x = hip.sparse_solve(pat, vals, b, method="bicgstab", precond="none", tol=1e-12, maxit=2000)
    loss = 0.5 * ((x - d["xt"]) ** 2).sum()
    loss.backward()
    r, a = oracle_forward_adjoint(p, tol=1e-12, maxit=2000)
    assert relerr(vals.grad.cpu().numpy(), a.grad_values) <= 1e-7
    assert relerr(b.grad.cpu().numpy(), a.grad_b) <= 1e-7
