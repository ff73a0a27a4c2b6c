"""Seeded synthetic inputs: CSR patterns, values, right-hand sides and loss targets.

This module only *builds problems*.  It contains no solver, no matrix-vector
product and no gradient: the oracle (``oracle/``) and the HIP library
(``differentiable_sparse_linear_amd``) both read the arrays produced here and
nothing else is shared between them.

Source of the workload family: the torch-sla explainer pages (gist.science,
"Technical summary", Results section) evaluate on a synthetic 2D Poisson
benchmark family only; no public dataset or suite is involved.  The five named
configurations widen that family (3D variable-coefficient diffusion, a batch of
shared-pattern systems, nonsymmetric convection-diffusion, and one GPU's share
of the pages' 4e8-unknown scale).  Readings used where the pages are silent:

* stencils are unscaled (no 1/h^2): 2D diagonal 4, neighbours -1;
* unknowns are numbered lexicographically with x fastest; columns ascend in each
  row, i.e. [-z, -y, -x, centre, +x, +y, +z];
* Dirichlet boundaries are eliminated: neighbours outside the grid are dropped
  and the diagonal keeps every face;
* variable coefficients: an interior face carries the harmonic mean
  2 k_a k_b / (k_a + k_b) of its two cells, a boundary face carries the cell's
  own k; diagonal = sum of all faces, off-diagonal = -face;
* convection-diffusion: first-order upwind with velocity (1, 0.5) and cell
  Peclet 10 measured with the max-norm of the velocity, scaled by h^2, giving
  diagonal 19, west -11, south -6, east -1, north -1;
* random draws use NumPy's PCG64 ``default_rng(seed)`` in the order
  kappa -> b -> x_t; batched arrays are drawn in one call, system-major;
* fp32 problems are built in fp64 and rounded to nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Problem",
    "laplacian_2d",
    "varcoef_diffusion",
    "upwind_convdiff_2d",
    "powerlaw_graph_laplacian",
    "random_csr",
    "config",
    "CONFIG_NAMES",
]


@dataclasses.dataclass
class Problem:
    """One workload: a CSR pattern shared by ``batch`` value arrays.

    row_ptr: int32 or int64 [n+1]; col: int32 [nnz] (ascending in each row);
    values: [batch, nnz] (float64 or float32); b, x_t: [batch, n].
    """

    name: str
    n: int
    row_ptr: np.ndarray
    col: np.ndarray
    values: np.ndarray
    b: np.ndarray
    x_t: np.ndarray
    method: str = "cg"          # "cg" | "bicgstab"
    precond: str = "jacobi"     # "none" | "jacobi"
    tol: float = 1e-10
    maxit: int = 1000
    grid: tuple = ()

    @property
    def nnz(self) -> int:
        return int(self.col.shape[0])

    @property
    def batch(self) -> int:
        return int(self.values.shape[0])

    @property
    def dtype(self):
        return self.values.dtype

    def astype(self, dtype) -> "Problem":
        """Round values, b and x_t to ``dtype`` (round-to-nearest-even)."""
        return dataclasses.replace(
            self,
            values=self.values.astype(dtype),
            b=self.b.astype(dtype),
            x_t=self.x_t.astype(dtype),
        )


# ----------------------------------------------------------------------------
# structured-grid stencils
# ----------------------------------------------------------------------------

def _grid_counts(dims: Sequence[int]) -> np.ndarray:
    """Entries per row (1 + number of in-grid neighbours), lexicographic order."""
    d = len(dims)
    cnt = np.ones(tuple(reversed(dims)), dtype=np.int8)
    for ax in range(d):
        # axis `ax` (0 = x) is the last numpy axis minus ax
        npax = d - 1 - ax
        size = dims[ax]
        shape = [1] * d
        shape[npax] = size
        inner = np.full(size, 2, dtype=np.int8)
        if size >= 1:
            inner[0] -= 1
            inner[-1] -= 1
        cnt = cnt + inner.reshape(shape)
    return cnt.reshape(-1)


def _row_ptr_from_counts(counts: np.ndarray, index_dtype) -> np.ndarray:
    rp = np.empty(counts.shape[0] + 1, dtype=np.int64)
    rp[0] = 0
    np.cumsum(counts, out=rp[1:])
    if index_dtype == np.int32:
        if rp[-1] >= 2**31:
            raise ValueError("nnz does not fit int32 row_ptr")
        return rp.astype(np.int32)
    return rp


def _assemble(dims, slot_fn, batch: int, index_dtype, value_dtype=np.float64,
              chunk_rows: int = 1 << 22):
    """Assemble a (2d+1)-slot stencil into CSR.

    ``slot_fn(lo, hi)`` returns (vals, mask) for rows [lo, hi): vals has shape
    [batch, hi-lo, 2d+1] (off-diagonal slots already negated, centre slot = the
    diagonal) and mask [hi-lo, 2d+1] marks in-grid neighbours.  Slots are in
    ascending column order.  Rows are processed in whole slowest-axis planes.
    """
    d = len(dims)
    n = int(np.prod(dims))
    counts = _grid_counts(dims)
    row_ptr = _row_ptr_from_counts(counts, index_dtype)
    nnz = int(row_ptr[-1])
    col = np.empty(nnz, dtype=np.int32)
    values = np.empty((batch, nnz), dtype=value_dtype)
    plane = int(np.prod(dims[:-1])) if d > 1 else n
    offs = []
    stride = 1
    strides = []
    for ax in range(d):
        strides.append(stride)
        stride *= dims[ax]
    for ax in reversed(range(d)):
        offs.append(-strides[ax])
    offs.append(0)
    for ax in range(d):
        offs.append(strides[ax])
    offs = np.asarray(offs, dtype=np.int64)
    planes_per_chunk = max(1, chunk_rows // plane)
    step = planes_per_chunk * plane

    def fill(lo):
        # chunks write disjoint slices, so they run on a thread pool (numpy
        # releases the GIL); the result does not depend on the order
        hi = min(n, lo + step)
        vals, mask = slot_fn(lo, hi)
        rows = np.arange(lo, hi, dtype=np.int64)
        cols = rows[:, None] + offs[None, :]
        s, e = int(row_ptr[lo]), int(row_ptr[hi])
        col[s:e] = cols[mask].astype(np.int32)
        for bi in range(batch):
            values[bi, s:e] = vals[bi][mask]

    starts = list(range(0, n, step))
    if len(starts) > 1:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, starts))
    else:
        for lo in starts:
            fill(lo)
    return row_ptr, col, values


def _neighbour_masks(dims, lo, hi):
    """mask[r, slot] for rows [lo, hi) (slot order -z,-y,-x,0,+x,+y,+z)."""
    d = len(dims)
    rows = np.arange(lo, hi, dtype=np.int64)
    coords = []
    rem = rows
    for ax in range(d):
        coords.append(rem % dims[ax])
        rem = rem // dims[ax]
    m = np.ones((hi - lo, 2 * d + 1), dtype=bool)
    for j, ax in enumerate(reversed(range(d))):
        m[:, j] = coords[ax] > 0
    for j, ax in enumerate(range(d)):
        m[:, d + 1 + j] = coords[ax] < dims[ax] - 1
    return m, coords


def laplacian_2d(N: int, index_dtype=np.int32):
    """Unscaled 5-point Dirichlet Laplacian on an N x N interior grid.

    Returns (row_ptr, col, values[1, nnz]); diagonal 4, neighbours -1.
    """
    dims = (N, N)

    def slot_fn(lo, hi):
        mask, _ = _neighbour_masks(dims, lo, hi)
        v = np.full((1, hi - lo, 5), -1.0)
        v[0, :, 2] = 4.0
        return v, mask

    return _assemble(dims, slot_fn, 1, index_dtype)


def _harm(a, b):
    # symmetric in (a, b) bit for bit: 2*a is exact and * and + commute
    return (2.0 * a * b) / (a + b)


def varcoef_diffusion(dims: Sequence[int], kappa: np.ndarray, index_dtype=np.int32,
                      chunk_rows: int = 1 << 22):
    """Cell-centred -div(k grad u) stencil, harmonic-mean faces, Dirichlet walls.

    dims = (Nx, Ny) or (Nx, Ny, Nz); kappa has shape [batch, n] or [n]
    (lexicographic, x fastest).  Interior face = harmonic mean of the two
    cells; a boundary face = the cell's own kappa; diagonal = sum of all 2d
    faces in slot order; off-diagonal = -face.  With kappa == 1 this is the
    unscaled constant-coefficient Laplacian.
    """
    dims = tuple(int(v) for v in dims)
    d = len(dims)
    kap = np.asarray(kappa, dtype=np.float64)
    if kap.ndim == 1:
        kap = kap[None, :]
    batch = kap.shape[0]
    n = int(np.prod(dims))
    assert kap.shape[1] == n
    strides = [int(np.prod(dims[:ax])) for ax in range(d)]

    def slot_fn(lo, hi):
        mask, coords = _neighbour_masks(dims, lo, hi)
        rows = np.arange(lo, hi, dtype=np.int64)
        kc = kap[:, lo:hi]
        v = np.empty((batch, hi - lo, 2 * d + 1))
        faces = {}
        for ax in range(d):
            st = strides[ax]
            # minus face
            nb = np.clip(rows - st, 0, n - 1)
            fm = np.where(coords[ax] > 0, _harm(kc, kap[:, nb]), kc)
            nb = np.clip(rows + st, 0, n - 1)
            fp = np.where(coords[ax] < dims[ax] - 1, _harm(kc, kap[:, nb]), kc)
            faces[(ax, -1)] = fm
            faces[(ax, +1)] = fp
        order = [(ax, -1) for ax in reversed(range(d))] + [(ax, +1) for ax in range(d)]
        diag = np.zeros_like(kc)
        for key in order:
            diag = diag + faces[key]
        for j, key in enumerate(order[:d]):
            v[:, :, j] = -faces[key]
        v[:, :, d] = diag
        for j, key in enumerate(order[d:]):
            v[:, :, d + 1 + j] = -faces[key]
        return v, mask

    return _assemble(dims, slot_fn, batch, index_dtype, chunk_rows=chunk_rows)


def upwind_convdiff_2d(N: int, velocity=(1.0, 0.5), peclet: float = 10.0,
                       index_dtype=np.int32):
    """First-order upwind -Lap(u) + (v/eps).grad(u) on N x N, scaled by h^2.

    Cell Peclet = max|v| h / eps.  For velocity (1, 0.5) and Peclet 10 this
    gives diagonal 19, west -11, south -6, east -1, north -1 (nonsymmetric,
    weakly diagonally dominant M-matrix).  Requires non-negative velocity.
    """
    vx, vy = velocity
    if vx < 0 or vy < 0:
        raise ValueError("only non-negative velocities are supported")
    vmax = max(abs(vx), abs(vy))
    cx, cy = peclet * vx / vmax, peclet * vy / vmax
    dims = (N, N)
    diag = 4.0 + cx + cy
    west, south = -1.0 - cx, -1.0 - cy

    def slot_fn(lo, hi):
        mask, _ = _neighbour_masks(dims, lo, hi)
        v = np.empty((1, hi - lo, 5))
        v[0, :, 0] = south
        v[0, :, 1] = west
        v[0, :, 2] = diag
        v[0, :, 3] = -1.0
        v[0, :, 4] = -1.0
        return v, mask

    return _assemble(dims, slot_fn, 1, index_dtype)


# ----------------------------------------------------------------------------
# irregular patterns (tests and the long-row SpMV)
# ----------------------------------------------------------------------------

def powerlaw_graph_laplacian(n: int, seed: int, avg_degree: int = 8,
                             alpha: float = 1.2, shift: float = 1.0):
    """Seeded weighted graph Laplacian + shift*I with a heavy-tailed degree mix.

    Edge endpoints are drawn with Zipf-like preference (weight ~ (rank+1)^-alpha
    over a random permutation), so a few rows are very long (thousands of
    entries) while most are short.  Edge weights ~ U[0.5, 1.5].  The result is
    symmetric positive definite (diagonal = weighted degree + shift).
    Returns (row_ptr int32, col int32, values[1, nnz] float64).
    """
    rng = np.random.default_rng(seed)
    m = n * avg_degree // 2
    w = (np.arange(n, dtype=np.float64) + 1.0) ** (-alpha)
    w /= w.sum()
    perm = rng.permutation(n)
    a = perm[rng.choice(n, size=m, p=w)]
    bnd = rng.integers(0, n, size=m)
    wt = rng.uniform(0.5, 1.5, size=m)
    keep = a != bnd
    a, bnd, wt = a[keep], bnd[keep], wt[keep]
    # dense-free assembly: sort (row, col) keys, merge duplicates by summation
    r = np.concatenate([a, bnd])
    c = np.concatenate([bnd, a])
    v = np.concatenate([wt, wt])
    key = r.astype(np.int64) * n + c
    order = np.argsort(key, kind="stable")
    key, v = key[order], v[order]
    uniq, start = np.unique(key, return_index=True)
    vsum = np.add.reduceat(v, start)
    r, c = uniq // n, uniq % n
    deg = np.bincount(r, weights=vsum, minlength=n)
    # insert diagonal entries
    r = np.concatenate([r, np.arange(n)])
    c = np.concatenate([c, np.arange(n)])
    vals = np.concatenate([-vsum, deg + shift])
    key = r * n + c
    order = np.argsort(key, kind="stable")
    r, c, vals = r[order], c[order], vals[order]
    counts = np.bincount(r, minlength=n)
    row_ptr = _row_ptr_from_counts(counts, np.int32)
    return row_ptr, c.astype(np.int32), vals[None, :]


def random_csr(n: int, density: float, seed: int, symmetric: bool = False,
               diag_dominant: bool = True, index_dtype=np.int32):
    """Small seeded random sparse matrix with every diagonal entry stored.

    Off-diagonal values ~ U[-1, 1]; with ``diag_dominant`` the diagonal is
    (row abs-sum + 1), making the matrix nonsingular (SPD when symmetric).
    Returns (row_ptr, col, values[1, nnz]) built from a dense mask, so use it
    for small n only.
    """
    rng = np.random.default_rng(seed)
    mask = rng.random((n, n)) < density
    vals = rng.uniform(-1.0, 1.0, (n, n))
    if symmetric:
        mask = mask | mask.T
        vals = np.triu(vals, 1)
        vals = vals + vals.T
    np.fill_diagonal(mask, True)
    dense = np.where(mask, vals, 0.0)
    np.fill_diagonal(dense, 0.0)
    if diag_dominant:
        np.fill_diagonal(dense, np.abs(dense).sum(axis=1) + 1.0)
    else:
        np.fill_diagonal(dense, rng.uniform(0.5, 1.5, n))
    rows, cols = np.nonzero(mask)
    counts = np.bincount(rows, minlength=n)
    row_ptr = _row_ptr_from_counts(counts, index_dtype)
    return row_ptr, cols.astype(np.int32), dense[rows, cols][None, :]


# ----------------------------------------------------------------------------
# the five named workloads (full size or scaled copies with the same recipe)
# ----------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "poisson2d_32x32_cg_fp64",
    2: "diffusion3d_100cubed_lognormal_jpcg_fp64",
    3: "batch1024_poisson2d_64x64_lognormal_jpcg",
    4: "convdiff2d_1024sq_upwind_bicgstab_fp64",
    5: "diffusion3d_512cubed_lognormal_jpcg_fp64",
}


def config(k: int, size: Optional[int] = None, batch: Optional[int] = None,
           dtype=np.float64, chunk_rows: int = 1 << 22) -> Problem:
    """Build workload ``k`` (1..5).

    ``size`` overrides the grid edge (same recipe and seed, scaled copy);
    ``batch`` overrides config 3's system count.  ``dtype`` float32 applies to
    config 3 (values built in fp64, then rounded).
    """
    rng = np.random.default_rng(k)
    if k == 1:
        N = size or 32
        rp, col, val = laplacian_2d(N)
        n = N * N
        b = rng.uniform(-1.0, 1.0, n)[None, :]
        xt = rng.uniform(-1.0, 1.0, n)[None, :]
        p = Problem(CONFIG_NAMES[1] if size is None else f"poisson2d_{N}x{N}_cg",
                    n, rp, col, val, b, xt, method="cg", precond="none",
                    tol=1e-10, maxit=10000, grid=(N, N))
    elif k == 2:
        N = size or 100
        n = N ** 3
        kap = np.exp(rng.standard_normal(n))
        rp, col, val = varcoef_diffusion((N, N, N), kap, chunk_rows=chunk_rows)
        b = rng.standard_normal(n)[None, :]
        xt = rng.uniform(-1.0, 1.0, n)[None, :]
        p = Problem(CONFIG_NAMES[2] if size is None else f"diffusion3d_{N}cubed_jpcg",
                    n, rp, col, val, b, xt, method="cg", precond="jacobi",
                    tol=1e-10, maxit=1000, grid=(N, N, N))
    elif k == 3:
        N = size or 64
        B = batch or 1024
        n = N * N
        kap = np.exp(0.5 * rng.standard_normal((B, n)))
        rp, col, val = varcoef_diffusion((N, N), kap)
        b = rng.standard_normal((B, n))
        xt = rng.uniform(-1.0, 1.0, (B, n))
        p = Problem(CONFIG_NAMES[3] if (size is None and batch is None)
                    else f"batch{B}_poisson2d_{N}x{N}_jpcg",
                    n, rp, col, val, b, xt, method="cg", precond="jacobi",
                    tol=1e-10, maxit=10000, grid=(N, N))
        if np.dtype(dtype) == np.float32:
            p = p.astype(np.float32)
            p.tol = 1e-5
            p.name += "_fp32"
    elif k == 4:
        N = size or 1024
        n = N * N
        rp, col, val = upwind_convdiff_2d(N)
        b = rng.standard_normal(n)[None, :]
        xt = rng.uniform(-1.0, 1.0, n)[None, :]
        p = Problem(CONFIG_NAMES[4] if size is None else f"convdiff2d_{N}sq_bicgstab",
                    n, rp, col, val, b, xt, method="bicgstab", precond="none",
                    tol=1e-10, maxit=2000, grid=(N, N))
    elif k == 5:
        N = size or 512
        n = N ** 3
        kap = np.exp(rng.standard_normal(n))
        rp, col, val = varcoef_diffusion((N, N, N), kap, index_dtype=np.int64,
                                         chunk_rows=chunk_rows)
        del kap
        b = rng.standard_normal(n)[None, :]
        xt = rng.uniform(-1.0, 1.0, n)[None, :]
        p = Problem(CONFIG_NAMES[5] if size is None else f"diffusion3d_{N}cubed_jpcg_i64",
                    n, rp, col, val, b, xt, method="cg", precond="jacobi",
                    tol=1e-10, maxit=500, grid=(N, N, N))
    else:
        raise ValueError(f"unknown workload {k}")
    return p
