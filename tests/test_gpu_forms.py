"""Which storage form the solver iterations pick, at the edges of the
diagonal-major form's eligibility (3, 5 or 7 diagonals, the main one in the
middle, at most 25 % padding), and parity with the oracle in each case.

Banded problems are built here from a list of diagonal offsets: row i stores
column i + d for every offset d that lands in [0, n).  Symmetric cases take
A_ij = A_ji = -(1 + sin(min(i, j) + |d|) / 2) off the diagonal and the
diagonal sum of the row's off-diagonal magnitudes plus 1/2 (strictly
diagonally dominant, hence SPD): CG with Jacobi.  Nonsymmetric cases scale the
entries above the diagonal by 0.6 and below by 1.4 (still diagonally
dominant): BiCGStab, whose adjoint iterates on the transposed pattern (the
negated offsets).  n = 5000 keeps every solve on the grid kernels.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import FP_TOL, banner, gpu_forward_adjoint, oracle_forward_adjoint, relerr

pytestmark = pytest.mark.gpu


def banded(name, n, offsets, symmetric, seed):
    offsets = sorted(offsets)
    rows, cols = [], []
    for d in offsets:
        i = np.arange(max(0, -d), min(n, n - d))
        rows.append(i)
        cols.append(i + d)
    rows = np.concatenate(rows)
    cols = np.concatenate(cols)
    order = np.lexsort((cols, rows))
    rows, cols = rows[order], cols[order]
    off = cols != rows
    v = np.zeros(rows.size)
    lo = np.minimum(rows, cols)
    dist = np.abs(cols - rows)
    v[off] = -(1.0 + 0.5 * np.sin(lo[off] + dist[off]))
    if not symmetric:
        v[off & (cols > rows)] *= 0.6
        v[off & (cols < rows)] *= 1.4
    diag = np.zeros(n)
    np.add.at(diag, rows[off], np.abs(v[off]))
    v[~off] = diag[rows[~off]] + 0.5
    row_ptr = np.zeros(n + 1, dtype=np.int32)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    rng = np.random.default_rng(seed)
    b = rng.standard_normal((1, n))
    xt = rng.uniform(-1.0, 1.0, (1, n))
    return W.Problem(name, n, row_ptr, cols.astype(np.int32), v[None, :], b, xt,
                     method="cg" if symmetric else "bicgstab",
                     precond="jacobi" if symmetric else "none", tol=1e-10, maxit=5000)


# (name, offsets, symmetric, the form the iterations read for A)
CASES = [
    ("tridiagonal", (-1, 0, 1), True, "diagonal-major"),
    ("tridiagonal_nonsym", (-1, 0, 1), False, "diagonal-major"),
    ("five_band", (-70, -1, 0, 1, 70), True, "diagonal-major"),
    ("five_band_nonsym", (-70, -1, 0, 1, 70), False, "diagonal-major"),
    ("upper_band", (0, 1, 2), False, "diagonal"),         # main diagonal not in the middle
    ("four_band", (-2, -1, 0, 1), False, "diagonal"),     # 4 diagonals
    ("wide_padding", (-4000, -1, 0, 1, 4000), True, "diagonal"),  # padding above 25 %
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_iteration_form_and_parity(hip, case):
    name, offsets, symmetric, form = case
    banner(f"forms: {name}")
    p = banded(name, 5000, offsets, symmetric, seed=len(name))
    g = gpu_forward_adjoint(hip, p)
    pat = g["pattern"]
    assert pat.column_mode() == "diagonal", name
    assert pat.iteration_form() == form, name
    if not symmetric:
        # A^T stores the negated offsets: the same eligibility
        assert pat.iteration_form(transpose=True) == form, name
    r, a = oracle_forward_adjoint(p)
    tol = FP_TOL[np.dtype(np.float64)]["sol"]
    assert g["info"]["status"][0] == 0 and r.status[0] == 0, (name, g["info"])
    assert g["ainfo"]["status"][0] == 0 and a.status[0] == 0, (name, g["ainfo"])
    assert relerr(g["x"][0], r.x[0]) <= tol, name
    assert relerr(g["gv"][0], a.grad_values[0]) <= tol, name
    assert relerr(g["gb"][0], a.grad_b[0]) <= tol, name
    assert abs(int(g["info"]["iters"][0]) - int(r.iters[0])) <= max(3, r.iters[0] // 50)


@pytest.mark.parametrize("case", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_diagonal_major_matches_csr_values_bitwise(hip, case):
    """The same solve and adjoint with the iterations on the caller's CSR
    values (SLA_CREATE_CSR_VALUES) give bitwise the same results."""
    import torch
    name, offsets, symmetric, form = case
    banner(f"forms bitwise: {name}")
    p = banded(name, 5000, offsets, symmetric, seed=len(name))
    outs = []
    for dmaj in (True, False):
        rp = torch.from_numpy(p.row_ptr).cuda()
        col = torch.from_numpy(p.col).cuda()
        val = torch.from_numpy(p.values).cuda()
        b = torch.from_numpy(p.b).cuda()
        xt = torch.from_numpy(p.x_t).cuda()
        pat = hip.Pattern(rp, col, build_transpose=not symmetric, diagonal_major=dmaj)
        assert pat.iteration_form() == ("diagonal-major" if dmaj else "diagonal")
        kw = dict(method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit)
        x, info = pat.solve(val, b, **kw)
        gv, gb, ainfo = pat.solve_adjoint(val, x, x - xt, **kw)
        # CG on symmetric values reads the lower diagonals through their mirrors
        want = ("diagonal-major-symmetric" if symmetric else "diagonal-major") if dmaj else "diagonal"
        assert info["form"] == want and ainfo["form"] == want, (name, info["form"], ainfo["form"])
        outs.append([t.cpu().numpy() for t in (x, gv, gb)] + [info["iters"], ainfo["iters"]])
        pat.close()
    for u, v in zip(outs[0], outs[1]):
        assert np.array_equal(np.asarray(u), np.asarray(v)), name


# A seven-band operator shaped like a 3D stencil on a 61 x 67 x 63 grid
# (offsets +-1, +-61, +-4087): too few planes per workgroup for the z-walk, so
# the iterations take the fast diagonal-major tiles, whose +-1 gathers come
# from the adjacent lanes and, for the lanes at a wavefront's edges, from
# scalar loads.  n = 257481 spans 1006 tiles (more than one per workgroup)
# and ends 201 rows into the last one, inside its fourth wavefront.  Past
# 768 tiles these solves launch 96 workgroups per XCD while the CSR-value
# iterations launch up to 128, so their partial sums are added in another
# order: the check is the oracle's iterates at fixed counts (every lane's
# neighbours enter from the first iteration on), and converged solves
# within rounding of each other.  The 5000-row cases above compare the same
# tiles with the CSR-value iterations bit for bit (one grid there).
FAST_OFFSETS = (-4087, -61, -1, 0, 1, 61, 4087)


def fast_problem(symmetric):
    return banded("seven_band", 61 * 67 * 63, FAST_OFFSETS, symmetric, seed=3)


@pytest.mark.parametrize("symmetric", [True, False], ids=["cg", "bicgstab"])
def test_fast_tiles_fixed_counts_match_oracle(hip, symmetric):
    """Forward and adjoint iterates after 1, 6 and 7 iterations (both
    parities of the CG kernel) on the fast tiles equal the oracle's to
    1e-12."""
    banner(f"forms: fast tiles at fixed counts {'cg' if symmetric else 'bicgstab'}")
    p = fast_problem(symmetric)
    form = "diagonal-major-symmetric" if symmetric else "diagonal-major"
    for k in (1, 6, 7):
        g = gpu_forward_adjoint(hip, p, maxit=k)
        assert g["info"]["form"] == g["ainfo"]["form"] == form, (g["info"]["form"], k)
        r, a = oracle_forward_adjoint(p, maxit=k)
        assert g["info"]["iters"][0] == r.iters[0], (k, g["info"]["iters"], r.iters)
        assert g["ainfo"]["iters"][0] == a.iters[0], (k, g["ainfo"]["iters"], a.iters)
        assert relerr(g["x"][0], r.x[0]) <= 1e-12, k
        assert relerr(g["gb"][0], a.grad_b[0]) <= 1e-12, k
        assert relerr(g["gv"][0], a.grad_values[0]) <= 1e-12, k
        g["pattern"].close()


@pytest.mark.parametrize("symmetric", [True, False], ids=["cg", "bicgstab"])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_fast_tiles_converge_with_csr_values(hip, dtype, symmetric):
    """Converged forward + adjoint on the fast tiles and on the caller's CSR
    values (diagonal masks, every gather loaded) agree within rounding: 1e-8
    in fp64 (tol 1e-10), 1e-4 in fp32 (tol 1e-5)."""
    import torch
    banner(f"forms: fast tiles converged {np.dtype(dtype).name} {'cg' if symmetric else 'bicgstab'}")
    p = fast_problem(symmetric)
    tol, agree = 1e-10, 1e-8
    if dtype == np.float32:
        p = p.astype(np.float32)
        tol, agree = 1e-5, 1e-4
    outs = []
    for dmaj in (True, False):
        rp = torch.from_numpy(p.row_ptr).cuda()
        col = torch.from_numpy(p.col).cuda()
        val = torch.from_numpy(p.values).cuda()
        b = torch.from_numpy(p.b).cuda()
        xt = torch.from_numpy(p.x_t).cuda()
        pat = hip.Pattern(rp, col, dtype=val.dtype, build_transpose=not symmetric,
                          diagonal_major=dmaj)
        kw = dict(method=p.method, precond=p.precond, tol=tol, maxit=p.maxit)
        x, info = pat.solve(val, b, **kw)
        gv, gb, ainfo = pat.solve_adjoint(val, x, x - xt, **kw)
        assert info["status"][0] == 0 and ainfo["status"][0] == 0, (info, ainfo)
        want = ("diagonal-major-symmetric" if symmetric else "diagonal-major") if dmaj else "diagonal"
        assert info["form"] == ainfo["form"] == want, (info["form"], ainfo["form"])
        outs.append([t.cpu().numpy().astype(np.float64) for t in (x, gv, gb)])
        pat.close()
    for u, v in zip(outs[0], outs[1]):
        assert relerr(u, v) <= agree


# Row pairs (fp64, n and the offsets other than +-1 even, more tiles than the
# grid's 768 workgroups): two consecutive rows per lane, 16-byte accesses.
# Five bands at +-1 and +-510 on n = 510 x 403 = 205530 rows (402 tiles of
# 512 rows, the last one 218 rows long, ending inside its second wavefront),
# CG on symmetric values and BiCGStab; seven bands shaped like a 62 x 64 x 67
# grid (+-1, +-62, +-3968; n = 265856, the last tile one wavefront long), CG.
# BiCGStab on seven diagonals keeps one row per lane (its pair kernel would
# spill), as does fp32.
PAIR_CASES = [
    ("five_band_cg", (-510, -1, 0, 1, 510), 510 * 403, True),
    ("five_band_bicgstab", (-510, -1, 0, 1, 510), 510 * 403, False),
    ("seven_band_cg", (-3968, -62, -1, 0, 1, 62, 3968), 62 * 64 * 67, True),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=[c[0] for c in PAIR_CASES])
def test_pair_tiles_fixed_counts_match_oracle(hip, case):
    """Forward and adjoint iterates after 1, 6 and 7 iterations on the row
    pair tiles equal the oracle's to 1e-12."""
    name, offsets, n, symmetric = case
    banner(f"forms: pair tiles at fixed counts {name}")
    p = banded(name, n, offsets, symmetric, seed=4)
    form = "diagonal-major-symmetric" if symmetric else "diagonal-major"
    for k in (1, 6, 7):
        g = gpu_forward_adjoint(hip, p, maxit=k)
        assert g["info"]["form"] == g["ainfo"]["form"] == form, (g["info"]["form"], k)
        r, a = oracle_forward_adjoint(p, maxit=k)
        assert g["info"]["iters"][0] == r.iters[0], (k, g["info"]["iters"], r.iters)
        assert g["ainfo"]["iters"][0] == a.iters[0], (k, g["ainfo"]["iters"], a.iters)
        assert relerr(g["x"][0], r.x[0]) <= 1e-12, k
        assert relerr(g["gb"][0], a.grad_b[0]) <= 1e-12, k
        assert relerr(g["gv"][0], a.grad_values[0]) <= 1e-12, k
        g["pattern"].close()


@pytest.mark.parametrize("case", PAIR_CASES, ids=[c[0] for c in PAIR_CASES])
def test_pair_tiles_converge_with_csr_values(hip, case):
    """Converged forward + adjoint on the row pair tiles and on the caller's
    CSR values (diagonal masks, one row per lane) agree to 1e-8 (tol 1e-10),
    and with the oracle's to the parity tolerance."""
    import torch
    name, offsets, n, symmetric = case
    banner(f"forms: pair tiles converged {name}")
    p = banded(name, n, offsets, symmetric, seed=4)
    outs = []
    for dmaj in (True, False):
        rp = torch.from_numpy(p.row_ptr).cuda()
        col = torch.from_numpy(p.col).cuda()
        val = torch.from_numpy(p.values).cuda()
        b = torch.from_numpy(p.b).cuda()
        xt = torch.from_numpy(p.x_t).cuda()
        pat = hip.Pattern(rp, col, build_transpose=not symmetric, diagonal_major=dmaj)
        kw = dict(method=p.method, precond=p.precond, tol=p.tol, maxit=p.maxit)
        x, info = pat.solve(val, b, **kw)
        gv, gb, ainfo = pat.solve_adjoint(val, x, x - xt, **kw)
        assert info["status"][0] == 0 and ainfo["status"][0] == 0, (info, ainfo)
        want = ("diagonal-major-symmetric" if symmetric else "diagonal-major") if dmaj else "diagonal"
        assert info["form"] == ainfo["form"] == want, (info["form"], ainfo["form"])
        outs.append([t.cpu().numpy() for t in (x, gv, gb)])
        pat.close()
    for u, v in zip(outs[0], outs[1]):
        assert relerr(u, v) <= 1e-8
    r, a = oracle_forward_adjoint(p)
    tol = FP_TOL[np.dtype(np.float64)]["sol"]
    assert relerr(outs[0][0], r.x[0]) <= tol
    assert relerr(outs[0][1], a.grad_values[0]) <= tol
    assert relerr(outs[0][2], a.grad_b[0]) <= tol


def test_unsymmetric_values_read_every_diagonal(hip):
    """CG on a mirrored pattern reads the lower diagonals through their
    mirrors only in systems whose values the pack finds symmetric bit for
    bit.  One launch group of three 5000-row five-band systems: symmetric;
    one pair one ulp apart; one pair of zeros with opposite signs.  Every
    system equals, bit for bit, the same solve on the caller's CSR values and
    the same system solved alone on the diagonal-major handle."""
    import torch
    banner("forms: unsymmetric values in a launch group")
    q = banded("five_band", 5000, (-70, -1, 0, 1, 70), True, seed=9)
    rows = np.repeat(np.arange(q.n), np.diff(q.row_ptr))
    pos = {(int(r), int(c)): k for k, (r, c) in enumerate(zip(rows, q.col))}
    vals = np.repeat(q.values, 3, axis=0)
    k_up, k_lo = pos[(1000, 1070)], pos[(1070, 1000)]
    vals[1, k_lo] = np.nextafter(vals[1, k_lo], 0.0)
    k_up, k_lo = pos[(2000, 2001)], pos[(2001, 2000)]
    vals[2, k_up], vals[2, k_lo] = 0.0, -0.0
    rng = np.random.default_rng(10)
    b = rng.standard_normal((3, q.n))
    xt = rng.uniform(-1.0, 1.0, (3, q.n))
    kw = dict(method="cg", precond="jacobi", tol=1e-10, maxit=5000)

    def run(dmaj, sys):
        rp = torch.from_numpy(q.row_ptr).cuda()
        col = torch.from_numpy(q.col).cuda()
        v = torch.from_numpy(np.ascontiguousarray(vals[sys])).cuda()
        bb = torch.from_numpy(np.ascontiguousarray(b[sys])).cuda()
        t = torch.from_numpy(np.ascontiguousarray(xt[sys])).cuda()
        pat = hip.Pattern(rp, col, batch=len(sys), diagonal_major=dmaj)
        x, info = pat.solve(v, bb, **kw)
        gv, gb, ainfo = pat.solve_adjoint(v, x, x - t, **kw)
        assert all(s == 0 for s in info["status"]) and all(s == 0 for s in ainfo["status"])
        out = [u.cpu().numpy() for u in (x, gv, gb)] + [info["iters"], ainfo["iters"]]
        pat.close()
        return out, info["form"], ainfo["form"]

    group, f, af = run(True, [0, 1, 2])
    assert f == af == "diagonal-major"  # not every system of the call is symmetric
    csr, f, af = run(False, [0, 1, 2])
    assert f == af == "diagonal"
    for u, v in zip(group, csr):
        assert np.array_equal(np.asarray(u), np.asarray(v))
    for s, want in ((0, "diagonal-major-symmetric"), (1, "diagonal-major"), (2, "diagonal-major")):
        alone, f, af = run(True, [s])
        assert f == af == want, (s, f, af)
        for u, v in zip(alone, group):
            assert np.array_equal(np.asarray(u)[0], np.asarray(v)[s]), s


def zwalk_problem(Z=16, seed=21, NX=512, NY=512):
    """Lognormal-kappa diffusion on an NX x NY x Z grid: seven diagonals
    with offsets 0, +-1, +-NX, +-NX*NY.  At 512 x 512 x 16 a plane is 1024
    columns of 256 rows, one per workgroup, each walked over all 16 planes
    (the tiles' order in rounds, so the partial sums are those of the other
    forms); at 90 x 90 x 520 a plane of 8100 rows is 31 columns of 254 rows
    and one of 226, each column's 520 planes cut into 32 segments of 16 or
    17."""
    rng = np.random.default_rng(seed)
    dims = (NX, NY, Z)
    n = NX * NY * Z
    kap = np.exp(rng.standard_normal(n))
    rp, col, val = W.varcoef_diffusion(dims, kap)
    b = rng.standard_normal(n)[None, :]
    xt = rng.uniform(-1.0, 1.0, n)[None, :]
    return W.Problem(f"diffusion_{NX}x{NY}x{Z}", n, rp, col, val, b, xt, method="cg",
                     precond="jacobi", tol=1e-10, maxit=1000)


def zwalk_plan(n, D):
    """The z-walk plan the library derives for a 3D seven-point operator
    (restated): columns of at most 256 rows, segments per column from the
    1024-workgroup grid, at least 16 planes per segment."""
    tiles = (n + 255) // 256
    grid = 8 * min(128, (tiles + 7) // 8)
    ncol = (D + 255) // 256
    tw = (D + ncol - 1) // ncol
    nseg = grid // ncol
    nz = n // D
    ok = nseg >= 1 and nz // nseg >= 16
    return ok, ncol, tw, nseg, nz


def test_zwalk_conditions_hold():
    """The patterns of zwalk_problem meet the z-walk's conditions, and the
    workloads of 100^3 (4 planes per segment) do not."""
    p = zwalk_problem()
    rows = np.repeat(np.arange(p.n, dtype=np.int64), np.diff(p.row_ptr))
    off = np.unique(p.col.astype(np.int64) - rows)
    assert list(off) == [-262144, -512, -1, 0, 1, 512, 262144]
    assert zwalk_plan(p.n, 262144) == (True, 1024, 256, 1, 16)
    assert zwalk_plan(90 * 90 * 520, 8100) == (True, 32, 254, 32, 520)
    assert zwalk_plan(10 ** 6, 10 ** 4)[0] is False
    assert zwalk_plan(512 ** 3, 512 ** 2) == (True, 1024, 256, 1, 512)


def test_zwalk_ragged_columns_and_segments(hip):
    """90 x 90 x 520 (4.2e6 rows): ragged columns and segments of 16 or 17
    planes.  Fixed iteration counts against the oracle's iterates; the
    converged forward + adjoint against the same solve on the caller's CSR
    values (a different order of the partial sums, so to the solve's
    precision, not bit for bit) and the oracle's true residuals."""
    import torch
    banner("z-walk: ragged columns and segments")
    p = zwalk_problem(Z=520, seed=23, NX=90, NY=90)
    for k in (1, 6, 7):
        g = gpu_forward_adjoint(hip, p, maxit=k)
        assert g["pattern"].iteration_form() == "diagonal-major"
        r, a = oracle_forward_adjoint(p, maxit=k)
        assert g["info"]["iters"][0] == k == r.iters[0]
        assert relerr(g["x"][0], r.x[0]) <= 1e-12, k
        assert relerr(g["gb"][0], a.grad_b[0]) <= 1e-12, k
        g["pattern"].close()
    outs = []
    for dmaj in (True, False):
        d = {k: torch.from_numpy(v).cuda() for k, v in
             (("rp", p.row_ptr), ("col", p.col), ("val", p.values), ("b", p.b), ("xt", p.x_t))}
        pat = hip.Pattern(d["rp"], d["col"], diagonal_major=dmaj)
        kw = dict(method="cg", precond="jacobi", tol=p.tol, maxit=p.maxit)
        x, info = pat.solve(d["val"], d["b"], **kw)
        gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **kw)
        assert info["status"][0] == 0 and ainfo["status"][0] == 0
        outs.append((x.cpu().numpy(), gv.cpu().numpy(), gb.cpu().numpy(), info, ainfo))
        pat.close()
    (x1, gv1, gb1, i1, a1), (x2, gv2, gb2, i2, a2) = outs
    assert i1["form"] == "diagonal-major-symmetric"
    assert abs(int(i1["iters"][0]) - int(i2["iters"][0])) <= 2
    assert relerr(x1, x2) <= 1e-8 and relerr(gb1, gb2) <= 1e-8 and relerr(gv1, gv2) <= 1e-8
    tr = O.true_relres(p.row_ptr, p.col, p.values, x1, p.b)[0]
    assert tr <= 10 * p.tol, tr


def test_zwalk_matches_oracle_iterates(hip):
    """Fixed iteration counts (even and odd stops) against the oracle's
    iterates, forward and adjoint."""
    banner("z-walk: fixed iterations")
    p = zwalk_problem()
    for k in (1, 6, 7):
        g = gpu_forward_adjoint(hip, p, maxit=k)
        assert g["pattern"].iteration_form() == "diagonal-major"
        r, a = oracle_forward_adjoint(p, maxit=k)
        assert g["info"]["iters"][0] == k == r.iters[0]
        assert relerr(g["x"][0], r.x[0]) <= 1e-12, k
        assert relerr(g["gb"][0], a.grad_b[0]) <= 1e-12, k
        assert relerr(g["gv"][0], a.grad_values[0]) <= 1e-12, k


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_zwalk_equals_csr_value_iterations_bitwise(hip, dtype):
    """A converged forward + adjoint with the z-walk equals, bit for bit, the
    same solve on the caller's CSR values (no diagonal-major form, no
    z-walk), in fp64 (tol 1e-10) and fp32 (tol 1e-5)."""
    import torch
    banner(f"z-walk: bitwise {np.dtype(dtype).name}")
    p = zwalk_problem()
    tol = 1e-10
    if dtype == np.float32:
        p = p.astype(np.float32)
        tol = 1e-5
    outs = []
    for dmaj in (True, False):
        rp = torch.from_numpy(p.row_ptr).cuda()
        col = torch.from_numpy(p.col).cuda()
        val = torch.from_numpy(p.values).cuda()
        b = torch.from_numpy(p.b).cuda()
        xt = torch.from_numpy(p.x_t).cuda()
        pat = hip.Pattern(rp, col, dtype=torch.from_numpy(p.values[:1, :1]).dtype,
                          diagonal_major=dmaj)
        kw = dict(method="cg", precond="jacobi", tol=tol, maxit=1000)
        x, info = pat.solve(val, b, **kw)
        gv, gb, ainfo = pat.solve_adjoint(val, x, x - xt, **kw)
        assert info["status"][0] == 0 and ainfo["status"][0] == 0
        if dmaj:  # the -D entries carried along the walk, the others mirrored
            assert info["form"] == ainfo["form"] == "diagonal-major-symmetric"
        outs.append([t.cpu().numpy() for t in (x, gv, gb)] + [info["iters"], ainfo["iters"]])
        pat.close()
        del rp, col, val, b, xt, x, gv, gb
        torch.cuda.empty_cache()
    for u, v in zip(outs[0], outs[1]):
        assert np.array_equal(np.asarray(u), np.asarray(v))
