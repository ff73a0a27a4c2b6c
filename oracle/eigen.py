"""Oracle for eigenvalues and their gradients -- TEST INFRASTRUCTURE ONLY
(same rules as the rest of ``oracle/``).

The torch-sla pages (gist.science explainer, Methodology section 1: .eigsh
in the autograd-aware API; section 2, eigenvalue problems) give the gradient
of an eigenvalue by the Hellmann-Feynman theorem, dlambda/dA_ij = v_i v_j,
an outer product on the stored pattern (v the unit eigenvector of a simple
eigenvalue of a symmetric A).

eigsh: the dense symmetric eigen-decomposition of the CSR matrix
(numpy.linalg.eigh used as one library step), so small systems only.
eig_grad: sum_q g_q v_q[row(k)] v_q[col(k)] for every stored entry k.
"""
from __future__ import annotations

import numpy as np


def dense(row_ptr, col, values):
    rp = np.asarray(row_ptr, dtype=np.int64)
    n = rp.shape[0] - 1
    A = np.zeros((n, n))
    for i in range(n):
        for k in range(rp[i], rp[i + 1]):
            A[i, col[k]] = values[k]
    return A


def eigsh(row_ptr, col, values, k=1, largest=False):
    """(evals [k], evecs [k, n]): ascending for the smallest, descending for
    the largest."""
    w, V = np.linalg.eigh(dense(row_ptr, col, np.asarray(values, dtype=np.float64)))
    idx = np.argsort(w)
    idx = idx[::-1][:k] if largest else idx[:k]
    return w[idx], V[:, idx].T.copy()


def eig_grad(row_ptr, col, evecs, g):
    """grad[k] = sum_q g[q] v_q[row(k)] v_q[col(k)]."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    n = rp.shape[0] - 1
    out = np.zeros(rp[-1])
    for i in range(n):
        for k in range(rp[i], rp[i + 1]):
            out[k] = sum(g[q] * evecs[q][i] * evecs[q][col[k]] for q in range(len(g)))
    return out
