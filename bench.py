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

``roofline`` describes the dominant kernel, timed live with HIP events that
the runtime records at the start and end of every launch (hipExtLaunchKernel,
on the stream the kernel runs on) in a separate, untimed step in the
library's profile mode.  For CG that is ``cg_iter_kernel``: one launch is one
whole PCG iteration, and ``achieved`` prices it at the method's algorithmic
bytes per PCG iteration (SpMV plus the textbook recurrence's 11 vector passes)
    nnz*(sv + 4) + (n + 1)*sr + 2*n*sv + 11*n*sv
(sv, sr: value and row-pointer widths; 9 passes without a preconditioner).
``kernel_bytes_per_launch`` is what the fused kernel itself must move: the
matrix once in the form the handle iterates on (CSR values with 4 bytes of
column per entry, 2 with its compact tile-relative copy, or 2 bytes per row
with its diagonal masks, plus row pointers; or the diagonal-major values,
nd * n * sv, for 3/5/7-diagonal stencils, (nd // 2 + 1) * n * sv when CG
found the values symmetric and read the lower diagonals through their
mirrors: the form the profiled solve reports) plus, on average over the two
iteration parities, 9 vectors (even launches read u, w, s, p and write p, s,
u, w; odd launches also read and write x).  For BiCGStab both kernels of an
iteration are timed; each launch is priced at half of one textbook BiCGStab
iteration, (2*(nnz*(sv + 4) + (n + 1)*sr) + 19*n*sv) / 2, and moves the
matrix plus 7.5 vectors on average (bicg_xpv reads s, t, p, v, x, rhat and
writes x, r, p, v; bicg_st reads r, v, rhat and writes s, t).
``traffic`` is the HBM bytes per launch measured with rocprofv3 counters
(FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
1 GiB copy) and stored under profiles/ with a hash of the kernel's sources;
it is null when no such record matches the sources being run.
``cpu_baseline`` times the oracle (plain fp64 C) on the host on one forward +
adjoint solve of the same arrays.

Counter and trace summaries (written under profiles/):
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run -- \
        python3 bench.py --kernel-only 2
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run -- \
        python3 bench.py --kernel-only 2
    python3 bench.py --summarize-counters OUT/pmc_fetch OUT/pmc_write
    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- \
        python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline
    python3 bench.py --summarize-trace OUT/trace
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "differentiable_sparse_linear_amd", "csrc")
CALIB_BYTES = 1 << 30  # the calibration copy reads and writes 1 GiB


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, help="named workload 1..5 (default 2)")
    ap.add_argument("--size", type=int, default=None, help="grid edge override (scaled copy)")
    ap.add_argument("--fp32", action="store_true",
                    help="fp32 values and vectors (dot products in fp64), tol 1e-5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-chunk", type=int, default=0)
    ap.add_argument("--kernel-only", type=int, default=0,
                    help="run this many steps and a 1 GiB calibration copy, nothing timed "
                         "(for counter collection)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of --kernel-only")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--op", default="solve",
                    choices=("solve", "matvec", "matvec_vjp", "inverse", "nonlinear", "eigsh"),
                    help="solve: the forward + adjoint step (default); matvec / matvec_vjp: "
                         "the differentiable product and its backward pass on the same "
                         "system, 100 x steps calls timed; inverse: kappa recovery through the "
                         "differentiable solve (64 x 64 grid, 8 forcings, 40 x steps Adam "
                         "steps); nonlinear: differentiable Newton solve of A u + c u^3 = f "
                         "on the workload's matrix; eigsh: its largest eigenpair by Lanczos "
                         "and the eigenvalue gradient")
    ap.add_argument("--graph", action="store_true",
                    help="with --op matvec / matvec_vjp: the seeded power-law graph Laplacian "
                         "(2^20 rows unless --size, seed 9; row lengths from 1 to 557 357) "
                         "instead of a numbered workload")
    ap.add_argument("--column-form", default="diagonal-major",
                    choices=("wide", "tile16", "diagonal", "diagonal-major",
                             "diagonal-major-symmetric"),
                    help="storage form the summarised run's iterations read")
    return ap.parse_args()


def dominant_kernel(method, precond, n, nnz, sv, sr, own_mat=None):
    """(kernel name(s), algorithmic bytes per launch, the kernel's own bytes
    per launch with `own_mat` bytes of matrix (default: CSR values, int32
    columns and row pointers), source files)."""
    mat = nnz * (sv + 4) + (n + 1) * sr
    own = mat if own_mat is None else own_mat
    if method == "cg":
        passes = 11 if precond == "jacobi" else 9
        return ("cg_iter_kernel", mat + (2 + passes) * n * sv, own + 9 * n * sv,
                ["kernels_cg.hip", "spmv_tile.h", "sla_internal.h"])
    # two launches per BiCGStab iteration: each is priced at half of one
    # textbook iteration (2 products + 19 vector passes)
    return ("bicg_xpv_kernel+bicg_st_kernel", (2 * mat + 19 * n * sv) // 2,
            own + (15 * n * sv) // 2, ["kernels_bicg.hip", "spmv_tile.h", "sla_internal.h"])


def num_diagonals(p):
    """Distinct column offsets col - row of the pattern."""
    rows = np.repeat(np.arange(p.n, dtype=np.int64), np.diff(p.row_ptr))
    return int(np.unique(p.col.astype(np.int64) - rows).size)


def form_bytes(form, p):
    """Bytes of the matrix one iteration product reads in `form`: CSR values
    plus int32 / int16 columns or one 16-bit diagonal mask per row plus the
    row pointers, or the diagonal-major values (padding included, no index)."""
    sv, sr = p.values.itemsize, p.row_ptr.itemsize
    if form == "diagonal-major":
        return num_diagonals(p) * p.n * sv
    if form == "diagonal-major-symmetric":  # the main and upper diagonals only
        return (num_diagonals(p) // 2 + 1) * p.n * sv
    idx = {"wide": 4 * p.nnz, "tile16": 2 * p.nnz, "diagonal": 2 * p.n}[form]
    return p.nnz * sv + idx + (p.n + 1) * sr


def sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}.{workload}.counters.txt")


def read_traffic(kernel, workload, sha):
    """HBM bytes per launch from a counter summary made from these sources, else None."""
    path = traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != sha:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def load_problem(args):
    import workloads as W
    if getattr(args, "graph", False):
        n = args.size or (1 << 20)
        rp, col, val = W.powerlaw_graph_laplacian(n, 9)
        return W.Problem(f"powerlaw_graph_{n}_seed9", n, rp, col, val, np.zeros((1, n)),
                         np.zeros((1, n)))
    if not getattr(args, "fp32", False):
        return W.config(args.workload, size=args.size)
    if args.workload == 3:
        return W.config(3, size=args.size, dtype=np.float32)
    p = W.config(args.workload, size=args.size).astype(np.float32)
    p.tol = 1e-5
    p.name += "_fp32"
    return p


# ------------------------------------------------------------------ summaries

def _rows(d, pattern):
    files = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _counter_pass(d, short_names):
    """(mean KiB of the active dominant-kernel dispatches, their count, all
    dispatches, KiB of the calibration copy)."""
    rows = _rows(d, "*counter_collection.csv")
    vals, copies = [], []
    for r in rows:
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if any(f"sla::{s}<" in name for s in short_names):
            vals.append(v)
        elif "copy" in name.lower() and "sla::" not in name:
            copies.append(v)
    if not vals or not copies:
        raise SystemExit(f"{d}: dominant kernel or calibration copy not found")
    # launches enqueued after the stop end at their first barrier and read a few bytes
    top = max(vals)
    active = [v for v in vals if v >= 0.01 * top]
    return sum(active) / len(active), len(active), len(vals), max(copies)


def _form_flag(args):
    return "" if args.column_form == "diagonal-major" else f" --column-form {args.column_form}"


def summarize_counters(args):
    p = load_problem(args)
    kernel, kbytes, own, srcs = dominant_kernel(p.method, p.precond, p.n, p.nnz,
                                                p.values.itemsize, p.row_ptr.itemsize,
                                                form_bytes(args.column_form, p))
    names = kernel.split("+")
    f_kib, f_n, f_all, f_copy = _counter_pass(args.summarize_counters[0], names)
    w_kib, w_n, w_all, w_copy = _counter_pass(args.summarize_counters[1], names)
    f_fac = CALIB_BYTES / (f_copy * 1024.0)
    w_fac = CALIB_BYTES / (w_copy * 1024.0)
    fetch = f_kib * 1024.0 * f_fac
    write = w_kib * 1024.0 * w_fac
    out = [
        f"# HBM traffic of {kernel}, workload {p.name}",
        "",
        "Commands (repository root; OUT is any output folder):",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run -- "
        f"python3 bench.py --kernel-only 2 --workload {args.workload}",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run -- "
        f"python3 bench.py --kernel-only 2 --workload {args.workload}",
        f"  python3 bench.py --summarize-counters OUT/pmc_fetch OUT/pmc_write --workload "
        f"{args.workload}{_form_flag(args)}",
        "",
        "Calibration: a torch copy of 1 GiB (reads 1 GiB, writes 1 GiB) in the same run;",
        "factor = 1 GiB / counter reading of that copy.",
        "",
        f"kernel: {kernel}",
        f"workload: {p.name}",
        f"n: {p.n}",
        f"nnz: {p.nnz}",
        f"source_sha256: {sources_sha(srcs)}",
        f"dispatches_active_fetch_pass: {f_n} of {f_all}",
        f"dispatches_active_write_pass: {w_n} of {w_all}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"copy_fetch_kib: {f_copy:.1f}",
        f"copy_write_kib: {w_copy:.1f}",
        f"fetch_factor: {f_fac:.4f}",
        f"write_factor: {w_fac:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"hbm_bytes_per_launch: {fetch + write:.0f}",
        f"algorithmic_bytes_per_launch: {kbytes}",
        f"kernel_bytes_per_launch: {own}",
        f"traffic_over_kernel_bytes: {(fetch + write) / own:.3f}",
    ]
    print("\n".join(out))


def summarize_trace(args):
    p = load_problem(args)
    kernel, kbytes, own, _ = dominant_kernel(p.method, p.precond, p.n, p.nnz,
                                             p.values.itemsize, p.row_ptr.itemsize,
                                             form_bytes(args.column_form, p))
    names = kernel.split("+")
    stats = _rows(args.summarize_trace, "*kernel_stats.csv")
    trace = _rows(args.summarize_trace, "*kernel_trace.csv")
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    op = "" if args.op == "solve" else f" --op {args.op}"
    which = " --graph" if args.graph else f" --workload {args.workload}"
    out = [
        f"# Kernel time, bench.py{op} on workload {p.name}",
        "",
        "Commands (repository root; OUT is any output folder):",
        "  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- "
        f"python3 bench.py{op} --steps 3 --warmup 1 --no-cpu-baseline{which}",
        f"  python3 bench.py --summarize-trace OUT/trace{op}{which}{_form_flag(args)}",
        "",
        "rocprofv3 --stats (all dispatches):",
        f"{'calls':>8} {'avg_us':>10} {'total_ms':>10} {'pct':>6}  kernel",
    ]
    for r in stats[:12]:
        name = r["Name"]
        short = name.split("(")[0].replace("void ", "")
        out.append(f"{int(r['Calls']):8d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['TotalDurationNs']) / 1e6:10.2f} {float(r['Percentage']):6.2f}  "
                   f"{short}")
    durs = []
    if args.op != "solve":
        names = []  # the per-kernel block below describes the solve's iteration kernel
    for r in trace:
        if any(f"sla::{s}<" in r["Kernel_Name"] for s in names):
            durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if durs:
        top = max(durs)
        # launches enqueued after the stop end at their first barrier (a few microseconds)
        active = [d for d in durs if d >= 0.25 * top]
        avg = sum(active) / len(active)
        out += [
            "",
            f"kernel: {kernel}",
            f"dispatches: {len(durs)}",
            f"dispatches_active: {len(active)} (the others ended at their first barrier after the stop)",
            f"avg_us_all: {sum(durs) / len(durs):.2f}",
            f"avg_us_active: {avg:.2f}",
            f"algorithmic_bytes_per_launch: {kbytes}",
            f"achieved_GBps_active: {kbytes / (avg * 1e-6) / 1e9:.1f}",
            f"kernel_bytes_per_launch: {own}",
            f"kernel_GBps_active: {own / (avg * 1e-6) / 1e9:.1f}",
        ]
    print("\n".join(out))


# ------------------------------------------------------------------ benchmark

def bench_nonlinear(args, p):
    """Differentiable Newton solve of A u + c u^3 = f (A the workload's
    matrix, c = 10, f its right-hand side) and the backward pass of
    L = 1/2 |u - x_t|^2 (one adjoint solve plus one vector-Jacobian product);
    `steps` forward + backward passes timed."""
    import torch
    import differentiable_sparse_linear_amd as sla
    from differentiable_sparse_linear_amd.nonlinear import Semilinear
    dev = "cuda:0"
    pat = sla.Pattern(torch.from_numpy(p.row_ptr).to(dev), torch.from_numpy(p.col).to(dev))
    model = Semilinear(pat)
    v = torch.from_numpy(p.values[0]).to(dev).requires_grad_(True)
    c = torch.full((p.n,), 10.0, dtype=torch.float64, device=dev, requires_grad=True)
    f = torch.from_numpy(p.b[0]).to(dev).requires_grad_(True)
    xt = torch.from_numpy(p.x_t[0]).to(dev)
    kw = dict(tol=1e-10, lin_tol=1e-10, lin_maxit=p.maxit, method=p.method, precond=p.precond)

    def step():
        u = model.solve(v, c, f, **kw)
        loss = 0.5 * torch.sum((u - xt) ** 2)
        loss.backward()
        return u.grad_fn.newton_iters, u.grad_fn.norms

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        its, norms = step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(json.dumps({
        "metric": "differentiable Newton solves/sec (forward + nonlinear adjoint)",
        "value": args.steps / wall, "unit": "solves/s", "n_gpus": 1, "steps": args.steps,
        "warmup": max(args.warmup, 1), "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (the workload's matrix and b, c = 10)",
        "config": {"workload": p.name + "_cubic", "n": p.n, "nnz": p.nnz,
                   "solver": f"newton+{p.method}+{p.precond}", "newton_tol": 1e-10},
        "newton_iters": its, "residual_norms": norms, "roofline": None,
    }), flush=True)


def bench_eigsh(args, p):
    """Largest eigenpair of the workload's matrix (Lanczos, 60-vector basis,
    tol 1e-8) and the gradient of the eigenvalue on the pattern; `steps`
    forward + backward passes timed."""
    import torch
    import differentiable_sparse_linear_amd as sla
    dev = "cuda:0"
    pat = sla.Pattern(torch.from_numpy(p.row_ptr).to(dev), torch.from_numpy(p.col).to(dev))
    v = torch.from_numpy(p.values[0]).to(dev).requires_grad_(True)
    opts = dict(k=1, largest=True, tol=1e-8, ncv=60, max_restarts=40)

    def step():
        v.grad = None
        ev, X = sla.sparse_eigsh(pat, v, **opts)
        ev.sum().backward()
        return ev

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _, _, info = pat.eigsh(v.detach(), **opts)
    print(json.dumps({
        "metric": "largest eigenpair + eigenvalue gradient per second", "value": args.steps / wall,
        "unit": "eigsh/s", "n_gpus": 1, "steps": args.steps, "warmup": max(args.warmup, 1),
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic (the workload's matrix)",
        "config": {"workload": p.name, "n": p.n, "nnz": p.nnz, "k": 1, "ncv": 60, "tol": 1e-8},
        "eigenvalue": float(ev.detach()[0, 0]), "restarts": int(info["restarts"][0]), "roofline": None,
    }), flush=True)


def bench_inverse(args):
    """Recover kappa = exp(theta) on a 64 x 64 grid from 8 observed solutions
    by Adam through the differentiable solve (forward and adjoint of 8
    systems per step, one workgroup per system)."""
    from differentiable_sparse_linear_amd import inverse as inv
    steps = 40 * max(args.steps, 1)
    inv.recover(N=64, B=8, steps=2)  # warm-up: library load, first launches
    out = inv.recover(N=64, B=8, steps=steps)
    print(json.dumps({
        "metric": "inverse-coefficient recovery, Adam steps/sec through the differentiable solve",
        "value": steps / out["wall_s"], "unit": "Adam steps/s", "n_gpus": 1, "steps": steps,
        "warmup": 2, "ms_per_step": out["wall_s"] * 1e3 / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (smooth log-kappa, 8 N(0,1) forcing fields, seed 11)",
        "config": {"workload": "inverse_kappa_64x64_b8", "grid": 64, "forcings": 8,
                   "lr": 0.05, "beta": 1e-6},
        "kappa_rel_err_start": out["kappa_rel_err_start"],
        "kappa_rel_err": out["kappa_rel_err"], "loss_first": out["loss"][0],
        "loss_last": out["loss"][-1], "wall_s": out["wall_s"], "roofline": None,
    }), flush=True)


def bench_product(args, p):
    """The differentiable product y = A x (matvec) or its backward pass
    (matvec_vjp: grad_x = A^T g and grad_values = g_i x_j) on the workload's
    matrix, `steps` calls timed with events on the stream they run on."""
    import torch
    import differentiable_sparse_linear_amd as sla
    dev = "cuda:0"
    tdt = torch.float64 if p.values.dtype == np.float64 else torch.float32
    rp = torch.from_numpy(p.row_ptr).to(dev)
    col = torch.from_numpy(p.col).to(dev)
    val = torch.from_numpy(p.values).to(dev)
    pat = sla.Pattern(rp, col, batch=p.batch, dtype=tdt, build_transpose=True)
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)).to(dev)
    g = torch.from_numpy(rng.standard_normal((p.batch, p.n)).astype(p.values.dtype)).to(dev)
    y = torch.empty_like(x)
    sv, sr = p.values.itemsize, p.row_ptr.itemsize
    # a pattern with rows past the tile walker's slots (the graph) also runs
    # the row plan's kernels
    plan = "+plan_spmv_kernel+plan_finish_kernel" if args.graph else ""
    if args.op == "matvec":
        call = lambda: pat.matvec(val, x, out=y)
        # values + columns + row pointers, x once, y written
        model = p.nnz * (sv + 4) + (p.n + 1) * sr + 2 * p.n * sv
        kernel = "spmv_kernel" + plan
    else:
        call = lambda: pat.matvec_adjoint(val, x, g)
        # values + columns + row pointers once, g, x read, grad_x and
        # grad_values written
        model = p.nnz * (2 * sv + 4) + (p.n + 1) * sr + 3 * p.n * sv
        # with diagonal masks one kernel makes both from A's own rows, else
        # A^T x goes through the transpose map and the gradient is a second
        # kernel
        kernel = ("diag_vjp_kernel" if pat.column_mode() == "diagonal"
                  else "spmv_perm_kernel+grad_kernel" + plan + ("+plan_grad_kernel" if plan else ""))
    model *= p.batch
    # a call takes tens of microseconds: enough calls that the timed region
    # spans milliseconds, after warm-up calls that bring the clocks up
    steps = max(args.steps, 1) * 100
    warm = max(args.warmup, 1) * 50
    for _ in range(warm):
        call()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = ev0.elapsed_time(ev1) / steps * 1e-3
    achieved = model / per / 1e9
    print(json.dumps({
        "metric": f"differentiable {args.op} calls/sec", "value": steps / wall,
        "unit": "calls/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": wall * 1e3 / steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64" if p.values.dtype == np.float64 else "f32",
        "data": "synthetic", "config": {"workload": p.name, "n": p.n, "nnz": p.nnz,
                                        "batch": p.batch},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "bytes_per_launch": model, "avg_launch_us": per * 1e6},
    }), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU "
              "sharding is a design note, not part of this build", file=sys.stderr)
        sys.exit(2)
    import torch
    import differentiable_sparse_linear_amd as sla

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    sla.load()
    if args.graph and args.op not in ("matvec", "matvec_vjp"):
        print("--graph is for --op matvec / matvec_vjp", file=sys.stderr)
        sys.exit(2)
    if args.op == "inverse":
        return bench_inverse(args)
    p = load_problem(args)
    if args.op == "nonlinear":
        return bench_nonlinear(args, p)
    if args.op == "eigsh":
        return bench_eigsh(args, p)
    if args.op != "solve":
        return bench_product(args, p)
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
        src = torch.empty(CALIB_BYTES // 8, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only, "calibration_copy_bytes": CALIB_BYTES}))
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
        # converged, or stopped at maxit (the 512^3 workload): no error, no breakdown
        assert np.all((info["status"] == 0) | (info["status"] == 1)), info

    block_path = p.method == "cg" and p.n <= 4096
    if block_path:
        roofline = None  # one workgroup per system: matrix in registers, vectors in LDS
    else:
        # dominant kernel, timed with HIP events around each launch on `stream`
        fi_p, ai_p = step(profile=True)
        torch.cuda.synchronize()
        k_ms = fi_p["kernel_ms"] + ai_p["kernel_ms"]
        k_n = fi_p["kernel_launches"] + ai_p["kernel_launches"]
        k_avg_s = (k_ms / k_n) * 1e-3 if k_n else float("nan")
        form = fi_p["form"]  # what the profiled iterations read
        fb = form_bytes(form, p)
        kernel, kbytes, own, srcs = dominant_kernel(p.method, p.precond, p.n, p.nnz,
                                                    p.values.itemsize, p.row_ptr.itemsize, fb)
        achieved = kbytes / k_avg_s / 1e9
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": read_traffic(kernel, p.name, sources_sha(srcs)),
                    "bytes_per_launch": kbytes, "kernel_bytes_per_launch": own,
                    "iteration_form": form, "kernel_GBps": own / k_avg_s / 1e9,
                    "avg_launch_us": k_avg_s * 1e6, "launches_timed": k_n}

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
        "data": f"synthetic (seeded workload {args.workload}: {p.name})",
        "config": {"workload": p.name, "n": p.n, "nnz": p.nnz, "batch": p.batch,
                   "solver": f"{p.method}+{p.precond}", "tol": p.tol, "maxit": p.maxit,
                   "iterations_per_step": iters / args.steps,
                   "forward_iters": int(fi["iters"].sum()), "adjoint_iters": int(ai["iters"].sum())},
        "solves_per_s": 2 * args.steps / wall,
        "event_ms_per_step": ev_ms / args.steps,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(result), flush=True)


def cpu_baseline(p, budget_s=15.0):
    """The oracle on a bounded sample of the same workload: whole forward +
    adjoint solves of the batch's systems in order until about `budget_s`
    seconds have passed (at least one); systems whose solve would take many
    minutes (n * maxit > 1e10, the 512^3 case) are cut to 5 iterations each
    way.  Rate in iterations (summed over systems) per second."""
    import oracle as O
    maxit = 5 if p.n * p.maxit > 1e10 else p.maxit
    t0 = time.perf_counter()
    its = systems = 0
    for s in range(p.batch):
        v = p.values[s].astype(np.float64)
        r = O.solve(p.row_ptr, p.col, v, p.b[s].astype(np.float64), p.method, p.precond,
                    p.tol, maxit)
        a = O.adjoint(p.row_ptr, p.col, v, r.x, r.x - p.x_t[s].astype(np.float64), p.method,
                      p.precond, p.tol, maxit)
        its += int(r.iters.sum() + a.iters.sum())
        systems += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t = time.perf_counter() - t0
    cut = f", cut to {maxit} iterations each way" if maxit != p.maxit else ""
    return {"value": its / t, "unit": "PCG iterations/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"forward + adjoint solves of {systems} of {p.batch} system(s) of {p.name}"
                      f"{cut} ({its} iterations, {t:.1f} s)"}


if __name__ == "__main__":
    main()
