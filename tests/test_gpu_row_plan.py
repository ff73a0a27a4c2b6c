"""Patterns with long rows: the row plan of the stand-alone products and the
gradient.

The backward pass and the A^T products of a single system (or of any batch
on a pattern of at least 2^20 entries) go in two passes: A's rows write the
terms v_k g_i in runs of A^T's rows, then A^T's rows are summed (each run
put back in A^T's order in LDS); smaller batches read A^T's values through
the transpose map (the 2^16-row batch of three).

Tiles whose entries exceed the tile walker's LDS stage, or that hold a row
longer than its gather slots, are covered by a plan built at set-up: short
blocks (rows of at most 64 entries, at most 2048 entries per block) and long
rows split into chunks of 2048 entries, one workgroup each, with a last pass
over the chunks of a split row.  Checked against the oracle: y = A x and
y = A^T x (fp64 and fp32, batches, int64 row pointers), the product's
backward pass, and a CG solve + adjoint whose gradient runs on the plan;
row lengths straddle the plan's limits (64 / 65 entries, 2048 / 2049, a row
of many chunks).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import FP_TOL, banner, oracle_forward_adjoint, relerr, tdtype, to_dev
from test_gpu_parity import _spmv_case, _vjp_case

pytestmark = pytest.mark.gpu


def lengths_pattern(n, base, special, seed, batch=1, dtype=np.float64, index=np.int32):
    """Rows of `base` entries each (a list, cycled over the rows) except the
    rows in `special` (row: length); every row holds its diagonal and
    distinct random columns, ascending."""
    rng = np.random.default_rng(seed)
    cols = []
    for i in range(n):
        L = min(special.get(i, base[i % len(base)]), n)
        other = rng.choice(n - 1, size=L - 1, replace=False)
        other = other + (other >= i)
        cols.append(np.sort(np.concatenate([other, [i]])))
    counts = np.array([c.size for c in cols])
    rp = np.zeros(n + 1, dtype=index)
    rp[1:] = np.cumsum(counts)
    col = np.concatenate(cols).astype(np.int32)
    val = rng.uniform(-1.0, 1.0, (batch, col.size)).astype(dtype)
    z = np.zeros((batch, n), dtype=dtype)
    return W.Problem(f"lengths_{n}_{seed}", n, rp, col, val, z, z)


def star_pattern(n, seed):
    """Row 0 holds every column (a row of n entries, several chunks); every
    other row holds its diagonal and column 0, so A^T's row 0 is full too."""
    rng = np.random.default_rng(seed)
    rows = [np.arange(n)] + [np.array([0, i]) for i in range(1, n)]
    counts = np.array([r.size for r in rows])
    rp = np.zeros(n + 1, dtype=np.int32)
    rp[1:] = np.cumsum(counts)
    col = np.concatenate(rows).astype(np.int32)
    val = rng.uniform(-1.0, 1.0, (1, col.size))
    z = np.zeros((1, n))
    return W.Problem(f"star_{n}", n, rp, col, val, z, z)


def circulant_pattern(n, stride, seed):
    """A circulant with columns (i + k * stride) mod n, k = 0..7, in row i,
    relabelled by one random permutation of rows and columns alike (the
    diagonal stays, the offsets scatter past any diagonal masks): every row
    and every column holds 8 entries, so A^T's tiles of 256 rows hold exactly
    2048 entries, the most the row sums stage whole (the last tile is
    ragged)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    cols = [None] * n
    for i in range(n):
        cols[perm[i]] = np.sort(perm[(i + stride * np.arange(8)) % n])
    rp = np.zeros(n + 1, dtype=np.int32)
    rp[1:] = np.cumsum([c.size for c in cols])
    col = np.concatenate(cols).astype(np.int32)
    val = rng.uniform(-1.0, 1.0, (1, col.size))
    z = np.zeros((1, n))
    return W.Problem(f"circulant_{n}", n, rp, col, val, z, z)


def powerlaw(n, seed, batch=1, dtype=np.float64, index=np.int32):
    rp, col, val = W.powerlaw_graph_laplacian(n, seed)
    rng = np.random.default_rng(seed + 1)
    vals = np.repeat(val, batch, axis=0) * rng.uniform(0.5, 1.5, (batch, 1))
    z = np.zeros((batch, n), dtype=dtype)
    return W.Problem(f"powerlaw_{n}", n, rp.astype(index), col, vals.astype(dtype), z, z)


CASES = {
    "powerlaw_2^18": lambda: powerlaw(1 << 18, 5),
    "powerlaw_2^16_batch3_fp32": lambda: powerlaw(1 << 16, 6, batch=3, dtype=np.float32),
    "powerlaw_2^16_int64": lambda: powerlaw(1 << 16, 7, index=np.int64),
    # A^T products in two passes one system after another (2.2e6 entries)
    "powerlaw_2^18_batch2": lambda: powerlaw(1 << 18, 8, batch=2),
    "powerlaw_2^16_fp32": lambda: powerlaw(1 << 16, 9, dtype=np.float32),
    # rows of 8 / 9 entries (the walker's slots), 64 / 65 (a short block's rows)
    "lengths_at_limits": lambda: lengths_pattern(9000, [3, 8, 9, 64, 65, 3, 3, 2, 1], {}, 3),
    # one chunk of 2048 exactly, one entry more, two chunks exactly, one
    # more, four exactly, four and one, six and one
    "chunk_edges": lambda: lengths_pattern(
        9000, [3, 5, 2],
        {1: 2048, 2: 2049, 5: 4096, 300: 4097, 301: 8192, 8000: 8193, 8999: 12289}, 4),
    "star_20000": lambda: star_pattern(20000, 8),
    "circulant_9000": lambda: circulant_pattern(9000, 1001, 12),
}


@pytest.mark.parametrize("case", list(CASES))
def test_spmv_both_directions(hip, case):
    banner(f"row plan spmv {case}")
    p = CASES[case]()
    _spmv_case(hip, p, transpose=False)
    _spmv_case(hip, p, transpose=True)


@pytest.mark.parametrize("case", ["powerlaw_2^16_batch3_fp32", "powerlaw_2^18_batch2",
                                  "powerlaw_2^16_fp32", "chunk_edges", "star_20000",
                                  "circulant_9000"])
def test_matvec_adjoint(hip, case):
    banner(f"row plan matvec adjoint {case}")
    _vjp_case(hip, CASES[case]())


def test_repeat_is_bitwise(hip):
    """The plan's sums run in a fixed order: repeated products agree bit for
    bit, and the backward pass's grad_x is the A^T product's bits whether or
    not grad_values is made in the same pass."""
    banner("row plan determinism")
    p = powerlaw(1 << 18, 5)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((1, p.n))).cuda()
    g = torch.from_numpy(rng.standard_normal((1, p.n))).cuda()
    y0, t0 = pat.matvec(d["val"], x), pat.matvec(d["val"], g, transpose=True)
    gv0, gx0 = pat.matvec_adjoint(d["val"], x, g)
    for _ in range(3):
        assert torch.equal(pat.matvec(d["val"], x), y0)
        assert torch.equal(pat.matvec(d["val"], g, transpose=True), t0)
        gv, gx = pat.matvec_adjoint(d["val"], x, g)
        assert torch.equal(gv, gv0) and torch.equal(gx, gx0)
    _, gx1 = pat.matvec_adjoint(d["val"], x, g, need_grad_values=False)
    gv1, _ = pat.matvec_adjoint(d["val"], x, g, need_grad_x=False)
    assert torch.equal(gx0, t0) and torch.equal(gx1, t0) and torch.equal(gv1, gv0)


def test_transposed_paths_agree_bitwise(hip):
    """A^T products go in two passes for a single system (the terms written
    in runs, then put back in A^T's order in LDS and summed) and through the
    transpose map for a batch on a small pattern: both round each term and
    add a row's terms in the same order, so they agree bit for bit.  On a
    2^21-row graph (1.75e7 entries) the product alone and the backward pass
    with both outputs give the same bits, and the product matches the
    oracle."""
    banner("A^T through the map and in two passes")
    # runs of A^T's rows of every kind: tiles the row sums stage whole, short
    # blocks and long-row chunks of A^T's row plan, tiles past the stage
    for name, p in (("powerlaw_2^16", powerlaw(1 << 16, 11, batch=2)),
                    ("chunk_edges", CASES["chunk_edges"]()),
                    ("star_20000", CASES["star_20000"]()),
                    ("lengths_at_limits", CASES["lengths_at_limits"]()),
                    ("circulant_9000", CASES["circulant_9000"]())):
        if p.batch == 1:  # a second system with its own values
            p = W.Problem(p.name, p.n, p.row_ptr, p.col,
                          np.concatenate([p.values, -0.5 * p.values]), np.zeros((2, p.n)),
                          np.zeros((2, p.n)))
        d = to_dev(p)
        one = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
        two = hip.Pattern(d["rp"], d["col"], batch=2, dtype=tdtype(p), build_transpose=True)
        rng = np.random.default_rng(4)
        g = torch.from_numpy(rng.standard_normal((2, p.n))).cuda()
        x = torch.from_numpy(rng.standard_normal((2, p.n))).cuda()
        yb = two.matvec(d["val"], g, transpose=True)
        _, gxb = two.matvec_adjoint(d["val"], x, g)
        for s in range(2):
            vs, gs = d["val"][s:s + 1].contiguous(), g[s:s + 1].contiguous()
            ys = one.matvec(vs, gs, transpose=True)
            _, gxs = one.matvec_adjoint(vs, x[s:s + 1].contiguous(), gs)
            assert torch.equal(ys[0], yb[s]) and torch.equal(gxs[0], gxb[s]), (name, s)
        one.close()
        two.close()

    banner("A^T in two passes, 2^21 rows")
    p = powerlaw(1 << 21, 13)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((1, p.n))).cuda()
    g = torch.from_numpy(rng.standard_normal((1, p.n))).cuda()
    yt = pat.matvec(d["val"], g, transpose=True)
    gv, gx = pat.matvec_adjoint(d["val"], x, g)
    assert torch.equal(gx, yt)
    rpt, ct, perm = O.transpose(p.n, p.row_ptr, p.col)
    vt = p.values[0].astype(np.float64)[perm]
    gh = g.cpu().numpy()[0]
    ref = O.spmv(rpt, ct, vt, gh)
    bound = FP_TOL[np.dtype(np.float64)]["spmv"] * O.spmv(rpt, ct, np.abs(vt), np.abs(gh)) + 1e-300
    assert np.all(np.abs(yt.cpu().numpy()[0] - ref) <= bound)
    pat.close()


def test_cg_solve_and_adjoint_on_graph(hip):
    """CG + Jacobi on the power-law graph Laplacian (+ I): the forward's A x0
    product and the adjoint's gradient on the pattern run on the plan."""
    banner("row plan solve + adjoint")
    rp, col, val = W.powerlaw_graph_laplacian(30000, 11)
    rng = np.random.default_rng(12)
    p = W.Problem("powerlaw_30000_solve", 30000, rp, col, val, rng.standard_normal((1, 30000)),
                  rng.uniform(-1.0, 1.0, (1, 30000)), method="cg", precond="jacobi", tol=1e-10,
                  maxit=2000)
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p))
    kw = dict(method="cg", precond="jacobi", tol=p.tol, maxit=p.maxit)
    x, info = pat.solve(d["val"], d["b"], **kw)
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **kw)
    r, a = oracle_forward_adjoint(p)
    tol = FP_TOL[np.dtype(np.float64)]["sol"]
    assert info["status"][0] == 0 and ainfo["status"][0] == 0
    assert relerr(x.cpu().numpy()[0], r.x[0]) <= tol
    assert relerr(gb.cpu().numpy()[0], a.grad_b[0]) <= tol
    assert relerr(gv.cpu().numpy()[0], a.grad_values[0]) <= tol
    # the gradient is -lambda_i x_j entry by entry from the GPU's own lambda and x
    lam, xs = gb.cpu().numpy()[0], x.cpu().numpy()[0]
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    assert np.array_equal(gv.cpu().numpy()[0], -(lam[rows] * xs[p.col]))
    # an initial guess: A x0 on the plan
    x0 = torch.from_numpy(rng.standard_normal((1, p.n))).cuda()
    x2, info2 = pat.solve(d["val"], d["b"], x0=x0, **kw)
    assert info2["status"][0] == 0
    assert relerr(x2.cpu().numpy()[0], r.x[0]) <= tol


@pytest.mark.parametrize("case", ["powerlaw_2^18", "star_20000", "chunk_edges"])
def test_setup_with_long_rows_bit_exact(hip, case):
    """Set-up of patterns with rows past 64 entries (checked entry by entry):
    the diagonal index and the transpose map equal the oracle's."""
    banner(f"row plan setup {case}")
    p = CASES[case]()
    rp, col, n = p.row_ptr, p.col, p.n
    st, dp = O.check_pattern(n, rp, col)
    assert st == O.OK
    rpt, ct, perm = O.transpose(n, rp, col)
    pat = hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda(),
                      build_transpose=True)
    g_dp, g_rpt, g_ct, g_perm = pat.export_pattern()
    assert np.array_equal(g_dp.cpu().numpy().astype(np.int64), dp)
    assert np.array_equal(g_rpt.cpu().numpy().astype(np.int64), rpt)
    assert np.array_equal(g_ct.cpu().numpy(), ct)
    assert np.array_equal(g_perm.cpu().numpy().astype(np.int64), perm)


def test_invalid_long_row_patterns_rejected(hip):
    """The entry-by-entry checks reject what the oracle rejects: columns out
    of order, repeated, out of range, and a row without its diagonal, in a
    pattern whose longest row is past 64 entries."""
    banner("row plan invalid patterns")
    p = CASES["lengths_at_limits"]()
    rp, col, n = p.row_ptr, p.col, p.n
    long_row = int(np.argmax(np.diff(rp)))
    k = int(rp[long_row]) + 10  # inside the long row
    one = next(i for i in range(n - 1) if rp[i + 1] - rp[i] == 1)  # a row of its diagonal only
    cases = []
    bad = col.copy(); bad[k], bad[k + 1] = bad[k + 1], bad[k]; cases.append(bad)
    bad = col.copy(); bad[k + 1] = bad[k]; cases.append(bad)
    bad = col.copy(); bad[int(rp[long_row + 1]) - 1] = n; cases.append(bad)
    bad = col.copy(); bad[int(rp[long_row])] = -1; cases.append(bad)
    bad = col.copy(); bad[int(rp[one])] = one + 1; cases.append(bad)
    for c in cases:
        assert O.check_pattern(n, rp, c)[0] == O.ERR_PATTERN
        with pytest.raises(hip.SlaError) as ei:
            hip.Pattern(torch.from_numpy(rp).cuda(), torch.from_numpy(c).cuda())
        assert ei.value.status == hip.SLA_ERR_PATTERN


def graph_problem(n, seed, batch=1, precond="jacobi"):
    rp, col, val = W.powerlaw_graph_laplacian(n, seed)
    rng = np.random.default_rng(seed + 100)
    vals = np.repeat(val, batch, axis=0) * rng.uniform(0.7, 1.3, (batch, 1))
    return W.Problem(f"graph_{n}_{seed}_b{batch}", n, rp, col, vals,
                     rng.standard_normal((batch, n)), rng.uniform(-1.0, 1.0, (batch, n)),
                     method="cg", precond=precond, tol=1e-10, maxit=2000)


@pytest.mark.parametrize("precond", ["jacobi", "none"])
def test_split_cg_matches_oracle_iterates(hip, precond):
    """CG on a pattern with a row plan runs three launches per iteration; at
    fixed iteration counts (even and odd stops) its iterates are the
    oracle's, forward and adjoint."""
    banner(f"split cg iterates {precond}")
    p = graph_problem(30000, 13, precond=precond)
    # The library's one-reduction arrangement and the oracle's textbook
    # recurrence give the same iterates in exact arithmetic; their rounding
    # differences grow like k * kappa * eps.  With Jacobi the operator is well
    # conditioned; without it this graph's kappa is about 2.4e4 (largest
    # eigenvalue 1.8e4 from the hubs' degrees, smallest 0.74), so 8
    # iterations allow ~2e-11.
    # grad_values = -lambda_i x_j inherits the bound through the pattern:
    # with |dx| <= tol |x| and |dlambda| <= tol |lambda| (asserted first),
    # |d(lambda_i x_j)| over the stored entries is at most
    # tol (|lambda|_inf sqrt(cmax) |x| + |x|_inf sqrt(rmax) |lambda|), rmax and
    # cmax the longest row and column (the hubs), plus one rounding per entry.
    tol = 1e-12 if precond == "jacobi" else 1e-10
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    rmax = int(np.diff(p.row_ptr).max())
    cmax = int(np.bincount(p.col, minlength=p.n).max())
    for k in (1, 2, 5, 8):
        g = _solve(hip, p, maxit=k)
        r, a = oracle_forward_adjoint(p, maxit=k)
        assert int(g["info"]["iters"][0]) == k == int(r.iters[0])
        assert relerr(g["x"][0], r.x[0]) <= tol, k
        assert relerr(g["gb"][0], a.grad_b[0]) <= tol, k
        xo, lo, gvo = r.x[0], a.grad_b[0], a.grad_values[0]
        gv_tol = tol * (np.abs(lo).max() * np.sqrt(cmax) * np.linalg.norm(xo) +
                        np.abs(xo).max() * np.sqrt(rmax) * np.linalg.norm(lo)) / \
            np.linalg.norm(gvo) + 4 * np.finfo(np.float64).eps
        assert relerr(g["gv"][0], gvo) <= gv_tol, (k, relerr(g["gv"][0], gvo), gv_tol)
        assert np.array_equal(g["gv"][0], -(g["gb"][0][rows] * g["x"][0][p.col])), k
    g = _solve(hip, p)
    r, a = oracle_forward_adjoint(p)
    sol = FP_TOL[np.dtype(np.float64)]["sol"]
    assert g["info"]["status"][0] == 0 and g["ainfo"]["status"][0] == 0
    assert relerr(g["x"][0], r.x[0]) <= sol and relerr(g["gv"][0], a.grad_values[0]) <= sol


def _solve(hip, p, profile=False, **kw):
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], batch=p.batch, dtype=tdtype(p))
    opts = dict(method="cg", precond=p.precond, tol=p.tol, maxit=p.maxit, check=False,
                profile=profile)
    opts.update(kw)
    x, info = pat.solve(d["val"], d["b"], **opts)
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **opts)
    torch.cuda.synchronize()
    out = dict(x=x.cpu().numpy(), gv=gv.cpu().numpy(), gb=gb.cpu().numpy(), info=info,
               ainfo=ainfo)
    pat.close()
    return out


def test_split_cg_batch_profile_and_edges(hip):
    """A batch of three graph systems (one launch group) equals the single
    solves bit for bit; profile mode (one system at a time, every iteration
    launched directly) gives the same results; a zero right-hand side and
    maxit = 0 stop at iteration 0."""
    banner("split cg batch / profile / edges")
    p = graph_problem(20000, 17, batch=3)
    g = _solve(hip, p)
    gp = _solve(hip, p, profile=True)
    for s in range(3):
        q = W.Problem("one", p.n, p.row_ptr, p.col, p.values[s:s + 1], p.b[s:s + 1],
                      p.x_t[s:s + 1], method="cg", precond="jacobi", tol=p.tol, maxit=p.maxit)
        gs = _solve(hip, q)
        for key in ("x", "gv", "gb"):
            assert np.array_equal(gs[key][0], g[key][s]), (s, key)
            assert np.array_equal(gp[key][s], g[key][s]), (s, key)
        assert gs["info"]["iters"][0] == g["info"]["iters"][s] == gp["info"]["iters"][s]
        assert g["info"]["status"][s] == 0 and g["ainfo"]["status"][s] == 0
    r, a = oracle_forward_adjoint(p, systems=[1])
    tol = FP_TOL[np.dtype(np.float64)]["sol"]
    assert relerr(g["x"][1], r.x[0]) <= tol and relerr(g["gv"][1], a.grad_values[0]) <= tol
    z = W.Problem("zero", p.n, p.row_ptr, p.col, p.values[:1], np.zeros((1, p.n)),
                  p.x_t[:1], method="cg", precond="jacobi", tol=p.tol, maxit=p.maxit)
    gz = _solve(hip, z)
    assert gz["info"]["iters"][0] == 0 and not np.any(gz["x"])
    g0 = _solve(hip, graph_problem(20000, 17), maxit=0)
    assert g0["info"]["iters"][0] == 0 and g0["info"]["status"][0] == hip.SLA_NOT_CONVERGED


def directed_graph_problem(n, seed):
    """The power-law graph with its entries above the diagonal scaled by 0.7
    and below by 1.3, the diagonal reset to the row's off-diagonal magnitude
    plus 1 (strictly diagonally dominant, nonsymmetric): BiCGStab."""
    rp, col, val = W.powerlaw_graph_laplacian(n, seed)
    rows = np.repeat(np.arange(n), np.diff(rp))
    v = val[0].copy()
    off = col != rows
    v[off & (col > rows)] *= 0.7
    v[off & (col < rows)] *= 1.3
    dsum = np.zeros(n)
    np.add.at(dsum, rows[off], np.abs(v[off]))
    v[~off] = dsum[rows[~off]] + 1.0
    rng = np.random.default_rng(seed + 200)
    return W.Problem(f"directed_graph_{n}_{seed}", n, rp, col, v[None, :],
                     rng.standard_normal((1, n)), rng.uniform(-1.0, 1.0, (1, n)),
                     method="bicgstab", precond="none", tol=1e-10, maxit=2000)


def _bsolve(hip, p, **kw):
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
    opts = dict(method="bicgstab", precond="none", tol=p.tol, maxit=p.maxit, check=False)
    opts.update(kw)
    x, info = pat.solve(d["val"], d["b"], **opts)
    gv, gb, ainfo = pat.solve_adjoint(d["val"], x, x - d["xt"], **opts)
    torch.cuda.synchronize()
    out = dict(x=x.cpu().numpy(), gv=gv.cpu().numpy(), gb=gb.cpu().numpy(), info=info,
               ainfo=ainfo)
    pat.close()
    return out


def test_split_bicgstab(hip):
    """BiCGStab on an operator with a row plan (A and, for the adjoint, A^T)
    runs six launches per iteration: the oracle's iterates at fixed counts,
    the converged forward and adjoint against the oracle, and profile mode
    and other chunk sizes (an odd one, made even) bit for bit the same."""
    banner("split bicgstab")
    p = directed_graph_problem(20000, 19)
    # the library's arrangement (one product and one set of partial sums per
    # half-iteration, rho from the identity rhat.(s - omega t) = rhat.s -
    # omega rhat.t) and the oracle's textbook steps agree in exact
    # arithmetic; rounding differences grow like k * kappa * eps, and this
    # operator's 2-norm condition number is about 1.9e4 (singular values
    # 1.9e4 and 0.99), so 5 iterations allow ~1e-11
    for k in (1, 2, 5):
        g = _bsolve(hip, p, maxit=k)
        r, a = oracle_forward_adjoint(p, maxit=k)
        assert int(g["info"]["iters"][0]) == k == int(r.iters[0]), k
        assert relerr(g["x"][0], r.x[0]) <= 1e-10, k
        assert relerr(g["gb"][0], a.grad_b[0]) <= 1e-10, k
    g = _bsolve(hip, p)
    r, a = oracle_forward_adjoint(p)
    sol = FP_TOL[np.dtype(np.float64)]["sol"]
    assert g["info"]["status"][0] == 0 and g["ainfo"]["status"][0] == 0
    assert relerr(g["x"][0], r.x[0]) <= sol
    assert relerr(g["gb"][0], a.grad_b[0]) <= sol
    assert relerr(g["gv"][0], a.grad_values[0]) <= sol
    # BiCGStab's residual history on this ill-conditioned operator is
    # erratic: the rounding differences above move the iteration at which it
    # first falls below the tolerance (both runs meet it; the solutions agree)
    assert abs(int(g["info"]["iters"][0]) - int(r.iters[0])) <= int(r.iters[0]) // 4
    for kw in ({"profile": True}, {"graph_chunk": 5}, {"graph_chunk": -6}):
        h = _bsolve(hip, p, **kw)
        for key in ("x", "gv", "gb"):
            assert np.array_equal(h[key], g[key]), (kw, key)
        assert h["info"]["iters"][0] == g["info"]["iters"][0], kw
    # an initial guess: A x0 through the plan
    d = to_dev(p)
    pat = hip.Pattern(d["rp"], d["col"], dtype=tdtype(p), build_transpose=True)
    x0 = torch.from_numpy(np.random.default_rng(3).standard_normal((1, p.n))).cuda()
    x, info = pat.solve(d["val"], d["b"], method="bicgstab", precond="none", tol=p.tol,
                        maxit=p.maxit, x0=x0)
    assert info["status"][0] == 0 and relerr(x.cpu().numpy()[0], r.x[0]) <= sol
