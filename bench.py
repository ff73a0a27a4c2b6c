#!/usr/bin/env python3
"""Benchmark: forward + adjoint Jacobi-PCG solve of the 1e6-DOF 3D
variable-coefficient diffusion system (100^3 cells, 6.94e6 stored entries,
fp64, tol 1e-10, maxit 1000) on one MI355X.

A step is one forward solve A x = b plus the adjoint backward pass
(A^T lambda = x - x_t, grad_b = lambda, grad_values on the pattern) -- the
whole differentiable solve.  Inputs are resident in HBM before timing starts.
Prints one JSON line.  ``value`` = PCG iterations per second (forward and
adjoint iterations summed over the timed steps, divided by the wall time
between the synchronised start and end).

``roofline`` describes the dominant kernel (the fused SpMV + direction update
of CG, ``cg_spmv_kernel``), timed live with HIP events on the stream it runs
on; its algorithmic bytes per launch are
    nnz*(8 + 4) + (n + 1)*4   matrix values, columns, row pointers
  + 2*n*8                     gathered z and previous p (each read once)
  + 2*n*8                     stored p and q.
``cpu_baseline`` times the oracle (plain fp64 C) on the host on one forward +
adjoint solve of the same arrays.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, help="named workload 1..5 (default 2)")
    ap.add_argument("--size", type=int, default=None, help="grid edge override (scaled copy)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-chunk", type=int, default=0)
    ap.add_argument("--kernel-only", type=int, default=0,
                    help="instead of the benchmark, launch the dominant kernel's solve this "
                         "many times (for counter collection)")
    return ap.parse_args()


def spmv_kernel_bytes(n, nnz, sv=8, sr=4):
    return nnz * (sv + 4) + (n + 1) * sr + 2 * n * sv + 2 * n * sv


def pcg_iteration_bytes(n, nnz, sv=8, sr=4):
    # fused SpMV kernel + update kernel (reads x, p, q, r, dinv; writes x, r, z)
    return spmv_kernel_bytes(n, nnz, sv, sr) + 5 * n * sv + 3 * n * sv


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU "
              "sharding is a design note, not part of this build", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import differentiable_sparse_linear_amd as sla

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    sla.load()
    p = W.config(args.workload, size=args.size)
    dev = "cuda:0"
    tdt = torch.float64 if p.values.dtype == np.float64 else torch.float32
    rp = torch.from_numpy(p.row_ptr).to(dev)
    col = torch.from_numpy(p.col).to(dev)
    val = torch.from_numpy(p.values).to(dev)
    b = torch.from_numpy(p.b).to(dev)
    xt = torch.from_numpy(p.x_t).to(dev)
    pat = sla.Pattern(rp, col, batch=p.batch, dtype=tdt, build_transpose=(p.method == "bicgstab"))
    opts = dict(tol=p.tol, maxit=p.maxit, method=p.method, precond=p.precond,
                graph_chunk=args.graph_chunk)
    x = torch.empty_like(b)
    gv = torch.empty_like(val)
    gb = torch.empty_like(b)
    stream = torch.cuda.current_stream()

    def step(profile=False):
        _, fi = pat.solve(val, b, out=x, profile=profile, **opts)
        g = x - xt
        _, _, ai = pat.solve_adjoint(val, x, g, out=(gv, gb), profile=profile, **opts)
        return fi, ai

    if args.kernel_only:
        for _ in range(args.kernel_only):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only}))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    iters = 0
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fi, ai = step()
        iters += int(fi["iters"].sum()) + int(ai["iters"].sum())
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    ev_ms = ev0.elapsed_time(ev1)
    for info in (fi, ai):
        assert np.all(info["status"] == 0), info

    # dominant kernel, timed with HIP events around each launch on `stream`
    fi_p, ai_p = step(profile=True)
    torch.cuda.synchronize()
    k_ms = fi_p["kernel_ms"] + ai_p["kernel_ms"]
    k_n = fi_p["kernel_launches"] + ai_p["kernel_launches"]
    k_avg_s = (k_ms / k_n) * 1e-3 if k_n else float("nan")
    kbytes = spmv_kernel_bytes(p.n, p.nnz, sv=p.values.itemsize, sr=p.row_ptr.itemsize) * p.batch
    achieved = kbytes / k_avg_s / 1e9

    iter_bytes = pcg_iteration_bytes(p.n, p.nnz, sv=p.values.itemsize, sr=p.row_ptr.itemsize)
    result = {
        "metric": "CG iters/sec + achieved HBM GB/s (% peak), fwd+adjoint solve, 1e6-DOF 3D Poisson",
        "value": iters / wall,
        "unit": "PCG iterations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if p.values.dtype == np.float64 else "f32",
        "data": "synthetic (seeded lognormal-coefficient 7-point diffusion, b ~ N(0,1))",
        "config": {"workload": p.name, "n": p.n, "nnz": p.nnz, "batch": p.batch,
                   "solver": f"{p.method}+{p.precond}", "tol": p.tol, "maxit": p.maxit,
                   "iterations_per_step": iters / args.steps,
                   "forward_iters": int(fi["iters"].sum()), "adjoint_iters": int(ai["iters"].sum())},
        "solves_per_s": 2 * args.steps / wall,
        "event_ms_per_step": ev_ms / args.steps,
        "model_iteration_bytes": iter_bytes,
        "model_iteration_GBps": iter_bytes * iters / wall / 1e9,
        "roofline": {"bound": "hbm", "kernel": "cg_spmv_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "bytes_per_launch": kbytes,
                     "avg_launch_us": k_avg_s * 1e6, "launches_timed": k_n},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        t0 = time.perf_counter()
        r = O.solve(p.row_ptr, p.col, p.values, p.b, p.method, p.precond, p.tol, p.maxit)
        a = O.adjoint(p.row_ptr, p.col, p.values, r.x, r.x - p.x_t, p.method, p.precond,
                      p.tol, p.maxit)
        t1 = time.perf_counter()
        oit = int(r.iters.sum() + a.iters.sum())
        result["cpu_baseline"] = {"value": oit / (t1 - t0), "unit": "PCG iterations/s",
                                  "cores": O.num_threads(), "kind": "oracle",
                                  "sample": f"one forward + adjoint solve of {p.name} "
                                            f"({oit} iterations, {t1 - t0:.1f} s)"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
