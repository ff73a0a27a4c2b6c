"""Write ``config5_maxit500.json``: the oracle's capped Jacobi-PCG forward
solve and adjoint on the 512^3 lognormal-coefficient diffusion system
(1.34e8 unknowns, int64 row pointers, tol 1e-10, maxit 500 -- the tolerance
is not reached, so both solves stop at the 500th iterate).

A capped solve has no closed form to compare with, so the full-size GPU
test compares the GPU's 500th iterates with the oracle's: this script stores
the oracle's iteration counts, statuses and recurrence residuals, the norms
of x and lambda, x and lambda at sampled rows, and the gradient on the
pattern at sampled stored entries.  Only ``oracle`` and ``workloads`` are
used.  Run from the repository root (about half an hour on 8 cores, 35 GB of
host memory):

    python3 tests/golden/make_config5_reference.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config5_maxit500.json")
ROW_SAMPLES, ENTRY_SAMPLES = 3000, 3000


def sample_rows(n):
    rng = np.random.default_rng(55)
    edge = [0, 1, 255, 256, n // 2, n - 257, n - 256, n - 2, n - 1]
    return np.unique(np.concatenate([rng.integers(0, n, ROW_SAMPLES), edge]))


def sample_entries(nnz):
    rng = np.random.default_rng(56)
    return np.unique(np.concatenate([rng.integers(0, nnz, ENTRY_SAMPLES), [0, 1, nnz - 1]]))


def main():
    t0 = time.time()
    p = W.config(5)
    print(f"generated {p.name} in {time.time() - t0:.0f} s", flush=True)
    t0 = time.time()
    r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, p.tol, p.maxit)
    print(f"forward: {r.iters[0]} iterations, status {r.status[0]}, relres {r.relres[0]:.6e}, "
          f"{time.time() - t0:.0f} s", flush=True)
    x = r.x[0]
    t0 = time.time()
    a = O.adjoint(p.row_ptr, p.col, p.values, r.x, r.x - p.x_t, p.method, p.precond, p.tol,
                  p.maxit)
    print(f"adjoint: {a.iters[0]} iterations, status {a.status[0]}, relres {a.relres[0]:.6e}, "
          f"{time.time() - t0:.0f} s", flush=True)
    lam = a.grad_b[0]
    rows = sample_rows(p.n)
    ents = sample_entries(p.nnz)
    true_rel = float(O.true_relres(p.row_ptr, p.col, p.values, r.x, p.b)[0])
    rec = {
        "workload": p.name, "n": p.n, "nnz": p.nnz, "method": p.method, "precond": p.precond,
        "tol": p.tol, "maxit": p.maxit,
        "forward": {"iters": int(r.iters[0]), "status": int(r.status[0]),
                    "relres": float(r.relres[0]), "true_relres": true_rel,
                    "norm": float(np.sqrt(O.dot(x, x)))},
        "adjoint": {"iters": int(a.iters[0]), "status": int(a.status[0]),
                    "relres": float(a.relres[0]), "norm": float(np.sqrt(O.dot(lam, lam)))},
        "rows": rows.tolist(),
        "x": [float(v) for v in x[rows]],
        "lambda": [float(v) for v in lam[rows]],
        "entries": ents.tolist(),
        "grad_values": [float(v) for v in a.grad_values[0][ents]],
    }
    with open(OUT, "w") as fh:
        json.dump(rec, fh, indent=0)
    print(f"wrote {OUT}", flush=True)


if __name__ == "__main__":
    main()
