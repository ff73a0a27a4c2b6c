"""Dense helpers for the oracle pins (NumPy only; independent of oracle.c)."""
import numpy as np


def to_dense(row_ptr, col, values):
    """Dense n x n matrix from CSR (one system)."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    n = rp.shape[0] - 1
    A = np.zeros((n, n))
    rows = np.repeat(np.arange(n), np.diff(rp))
    A[rows, np.asarray(col, dtype=np.int64)] = np.asarray(values, dtype=np.float64).reshape(-1)
    return A


def pattern_rows(row_ptr):
    rp = np.asarray(row_ptr, dtype=np.int64)
    return np.repeat(np.arange(rp.shape[0] - 1), np.diff(rp))


def laplacian_eigvec_2d(N, j, k):
    """Closed-form eigenvector of the unscaled 2D Dirichlet Laplacian (x fastest)."""
    p = np.arange(1, N + 1)
    h = np.pi / (N + 1)
    vx = np.sin(j * p * h)
    vy = np.sin(k * p * h)
    return np.outer(vy, vx).reshape(-1)


def laplacian_eigval_2d(N, j, k):
    h = np.pi / (N + 1)
    return 4.0 - 2.0 * np.cos(j * h) - 2.0 * np.cos(k * h)
