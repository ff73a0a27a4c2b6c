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
``traffic`` is the bytes per launch past L2 (to HBM or the Infinity Cache)
measured with rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each scaled by
what the counter reads for the probe library's 1 GiB copy; a third pass of
the read-request-size counters checks the scaled FETCH_SIZE without any
factor) and stored under profiles/ with a hash of the kernel's sources; it is
null when no such record matches the sources being run.  ``dram_GBps`` and
``dram_frac`` are that traffic over the average launch time; ``model_frac``
(= ``frac``) and ``kernel_frac`` price the launch at the textbook and the
fused kernel's own bytes.  ``ceilings`` are the chip's streaming and LDS
bandwidths measured in the same run by libsla_probe.so over 2 GiB arrays
(beyond the 256 MB Infinity Cache) and, as ``*_in_cache``, over 64 MiB
arrays that stay in it; ``dram_frac_of_copy_ceiling`` and
``dram_frac_of_in_cache_copy_ceiling`` set the traffic against the two
copies, and ``dram_frac_of_in_cache_stream_ceiling`` against launches of
pure in-cache streams shaped like the CG iteration (8 MB arrays, 8 read and
4 written, 9 and 5; ``streams_GBps_in_cache`` lists every shape measured);
for a working set beyond the cache (512^3) ``streams_GBps_hbm`` gives the
8 + 4 and 9 + 5 launches over 1 GiB arrays and
``dram_frac_of_hbm_stream_ceiling`` the traffic against them.
On the one-workgroup solver (at most 4096 rows) the roofline is LDS
bandwidth: (S + 11) values per row and iteration (S the gather slots).
``memory`` is the device memory of one forward + adjoint step.
``cpu_baseline`` times the oracle (plain fp64 C) on the host on bounded
samples of the same arrays, on all host threads and on one.

Counter and trace summaries (written under profiles/):
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run -- \
        python3 bench.py --kernel-only 2
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run -- \
        python3 bench.py --kernel-only 2
    rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum \
        TCC_EA0_RDREQ_128B_sum --output-format csv -d OUT/pmc_sizes -o run -- \
        python3 bench.py --kernel-only 2
    python3 bench.py --summarize-counters OUT/pmc_fetch OUT/pmc_write OUT/pmc_sizes
    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- \
        python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline
    python3 bench.py --summarize-trace OUT/trace
"""
import argparse
import csv
import ctypes
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
# LDS: 256 compute units x 256 bytes per clock x 2.4 GHz (CDNA4 doubled the
# 128 bytes per clock of CDNA3; the probe's ds_read_b128 stream sustains 140
# TB/s, above what 128 bytes per clock could deliver)
LDS_PEAK_GBPS = 256 * 256 * 2.4
LDS_PEAK_CU_GBPS = 256 * 2.4  # one compute unit
CSRC = os.path.join(ROOT, "differentiable_sparse_linear_amd", "csrc")
PROBE_LIB = os.path.join(ROOT, "differentiable_sparse_linear_amd", "libsla_probe.so")
CALIB_BYTES = 1 << 30  # the calibration kernels move 1 GiB each way
CEIL_BYTES = 2 << 30   # arrays of the ceiling measurement (beyond the 256 MB Infinity Cache)
CACHE_CEIL_BYTES = 64 << 20  # arrays of the in-cache ceilings (a copy touches 128 MiB)
# request-size counters of the optional third counter pass (bytes per request)
SIZE_COUNTERS = {"TCC_EA0_RDREQ_32B_sum": 32, "TCC_EA0_RDREQ_64B_sum": 64,
                 "TCC_EA0_RDREQ_128B_sum": 128}


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
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="summarise the rocprofv3 --pmc runs of --kernel-only: FETCH_SIZE, "
                         "WRITE_SIZE and optionally the read-request sizes")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-block", metavar="PMC_DIR",
                    help="summarise a rocprofv3 --pmc run of the one-workgroup solver's LDS "
                         "counters (workloads of at most 4096 rows)")
    ap.add_argument("--op", default="solve",
                    choices=("solve", "matvec", "matvec_t", "matvec_vjp", "inverse", "nonlinear",
                             "eigsh"),
                    help="solve: the forward + adjoint step (default); matvec / matvec_t / "
                         "matvec_vjp: the differentiable product, the A^T product alone and "
                         "the product's backward pass on the same system, 100 x steps calls "
                         "timed; inverse: kappa recovery through the "
                         "differentiable solve (64 x 64 grid, 8 forcings, 40 x steps Adam "
                         "steps); nonlinear: differentiable Newton solve of A u + c u^3 = f "
                         "on the workload's matrix; eigsh: its largest eigenpair by Lanczos "
                         "and the eigenvalue gradient")
    ap.add_argument("--graph", action="store_true",
                    help="with --op matvec / matvec_t / matvec_vjp: the seeded power-law graph "
                         "Laplacian "
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


def read_product_traffic(op, workload, sha):
    """Bytes past L2 per call of the product (op matvec) or its backward pass
    (matvec_vjp) from a counter summary under profiles/ made from these
    sources, else None."""
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*.{workload}.counters.txt"))):
        rec = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    rec[k.strip()] = v.strip()
        if rec.get("op") == op and rec.get("source_sha256") == sha:
            try:
                return float(rec["bytes_past_l2_per_call"])
            except (KeyError, ValueError):
                return None
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

def _short(name):
    """A kernel's name without its parameter list (and without the return
    type and anonymous-namespace prefixes)."""
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def _rows(d, pattern):
    files = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _dispatches(d):
    """Counter rows of a --pmc run grouped by dispatch: [(kernel name,
    {counter: value})] in dispatch order."""
    rows = _rows(d, "*counter_collection.csv")
    by = {}
    for r in rows:
        e = by.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], {}])
        e[1][r["Counter_Name"]] = e[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [tuple(by[k]) for k in sorted(by)]


def _is_probe(name, which):
    return f"::{which}_kernel(" in name and "sla::" not in name


def _pass_stats(d, short_names, counter):
    """(mean of `counter` over the active dominant-kernel dispatches, their
    count, all its dispatches, {probe: value} of the calibration kernels)."""
    vals, probes = [], {}
    for name, c in _dispatches(d):
        if counter not in c:
            continue
        if any(f"sla::{s}<" in name for s in short_names):
            vals.append(c[counter])
        for which in ("copy", "read", "write"):
            if _is_probe(name, which):
                probes[which] = max(probes.get(which, 0.0), c[counter])
    if not vals or "copy" not in probes:
        raise SystemExit(f"{d}: dominant kernel or calibration copy not found")
    # launches enqueued after the stop end at their first barrier and read a few bytes
    top = max(vals)
    active = [v for v in vals if v >= 0.01 * top]
    return sum(active) / len(active), len(active), len(vals), probes


def _size_stats(d, short_names):
    """Read bytes by request size (32, 64, 128 B) per active dominant-kernel
    dispatch and for the calibration kernels."""
    ker, probes = [], {}
    for name, c in _dispatches(d):
        if not all(k in c for k in SIZE_COUNTERS):
            continue
        by = sum(c[k] * sz for k, sz in SIZE_COUNTERS.items())
        if any(f"sla::{s}<" in name for s in short_names):
            ker.append(by)
        for which in ("copy", "read"):
            if _is_probe(name, which):
                probes[which] = max(probes.get(which, 0.0), by)
    top = max(ker)
    active = [v for v in ker if v >= 0.01 * top]
    return sum(active) / len(active), probes


def _form_flag(args):
    return "" if args.column_form == "diagonal-major" else f" --column-form {args.column_form}"


PRODUCT_KERNELS = ("spmv_kernel", "plan_spmv_kernel", "plan_finish_kernel",
                   "plan_grad_kernel", "grad_kernel", "rowsum_kernel", "diag_vjp_kernel")
CACHE_COUNTERS = ("TCC_HIT_sum", "TCC_MISS_sum", "TCP_TCC_READ_REQ_sum",
                  "TCP_TOTAL_CACHE_ACCESSES_sum")


def product_model_bytes(op, p):
    """Algorithmic bytes of one call of the product (op matvec), of the A^T
    product (matvec_t, the same bytes: values and columns once, one vector
    read, one written) or of the product's backward pass (matvec_vjp:
    grad_x = A^T g and grad_values)."""
    sv, sr = p.values.itemsize, p.row_ptr.itemsize
    if op in ("matvec", "matvec_t"):
        return (p.nnz * (sv + 4) + (p.n + 1) * sr + 2 * p.n * sv) * p.batch
    return (p.nnz * (2 * sv + 4) + (p.n + 1) * sr + 3 * p.n * sv) * p.batch


def _product_table(d, counter, calls):
    """{kernel (name with template arguments): (dispatches, mean of
    `counter` per dispatch, total per call)} over the product's kernels,
    and the calibration probes' readings."""
    per, probes = {}, {}
    for name, c in _dispatches(d):
        for which in ("copy", "read", "write"):
            if _is_probe(name, which) and counter in c:
                probes[which] = max(probes.get(which, 0.0), c[counter])
        short = _short(name)
        if counter not in c or not any(f"sla::{k}<" in name for k in PRODUCT_KERNELS):
            continue
        e = per.setdefault(short, [0, 0.0])
        e[0] += 1
        e[1] += c[counter]
    return {k: (n, v / n, v / calls) for k, (n, v) in per.items()}, probes


def summarize_product_counters(args):
    """Bytes past L2 of the product or its backward pass, per kernel and
    per call, from the --pmc runs of bench.py --op OP --kernel-only K
    (10 K calls): FETCH_SIZE, WRITE_SIZE, optionally the read-request sizes
    and the L2 / L1 hit counters."""
    p = load_problem(args)
    dirs = args.summarize_counters
    if len(dirs) not in (2, 3, 4):
        raise SystemExit("--summarize-counters FETCH_DIR WRITE_DIR [SIZES_DIR [CACHE_DIR]]")
    calls = 20
    which = (" --graph" + (f" --size {args.size}" if args.size else "") if args.graph
             else f" --workload {args.workload}")
    run = f"python3 bench.py --op {args.op} --kernel-only 2{which}"
    fetch, f_pr = _product_table(dirs[0], "FETCH_SIZE", calls)
    write, w_pr = _product_table(dirs[1], "WRITE_SIZE", calls)
    f_fac = CALIB_BYTES / (f_pr["copy"] * 1024.0)
    w_fac = CALIB_BYTES / (w_pr["copy"] * 1024.0)
    model = product_model_bytes(args.op, p)
    out = [
        f"# Bytes past L2 of the {args.op} call, workload {p.name}",
        "",
        "Commands (repository root; OUT is any output folder):",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run -- {run}",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run -- {run}",
        "  rocprofv3 --pmc " + " ".join(["TCC_EA0_RDREQ_sum"] + list(SIZE_COUNTERS)) +
        f" --output-format csv -d OUT/pmc_sizes -o run -- {run}",
        "  rocprofv3 --pmc " + " ".join(CACHE_COUNTERS) +
        f" --output-format csv -d OUT/pmc_cache -o run -- {run}",
        f"  python3 bench.py --op {args.op}{which} --summarize-counters OUT/pmc_fetch "
        "OUT/pmc_write OUT/pmc_sizes OUT/pmc_cache",
        "",
        f"The run makes {calls} calls, then the probe library's 1 GiB copy, read and write;",
        "FETCH_SIZE and WRITE_SIZE are scaled by 1 GiB over their reading of the copy.",
        "",
        f"op: {args.op}",
        f"workload: {p.name}",
        f"n: {p.n}",
        f"nnz: {p.nnz}",
        f"source_sha256: {sources_sha(['kernels_spmv.hip', 'spmv_tile.h', 'sla_internal.h'])}",
        f"fetch_factor: {f_fac:.4f}",
        f"write_factor: {w_fac:.4f}",
        f"algorithmic_bytes_per_call: {model}",
        "",
        f"{'dispatches':>10} {'fetch_MB':>10} {'write_MB':>10}  kernel (per dispatch, scaled)",
    ]
    tot_f = tot_w = 0.0
    for k in sorted(fetch, key=lambda k: -fetch[k][2]):
        n, fk, fc = fetch[k]
        wk = write.get(k, (0, 0.0, 0.0))
        out.append(f"{n:10d} {fk * 1024 * f_fac / 1e6:10.2f} {wk[1] * 1024 * w_fac / 1e6:10.2f}  {k}")
        tot_f += fc * 1024 * f_fac
        tot_w += wk[2] * 1024 * w_fac
    out += [
        "",
        f"fetch_bytes_per_call: {tot_f:.0f}",
        f"write_bytes_per_call: {tot_w:.0f}",
        f"bytes_past_l2_per_call: {tot_f + tot_w:.0f}",
        f"traffic_over_algorithmic_bytes: {(tot_f + tot_w) / model:.3f}",
    ]
    if len(dirs) >= 3:
        sized = {}
        for name, c in _dispatches(dirs[2]):
            if not all(k in c for k in SIZE_COUNTERS):
                continue
            short = _short(name)
            if any(f"sla::{k}<" in name for k in PRODUCT_KERNELS):
                e = sized.setdefault(short, [0, 0.0, [0.0, 0.0, 0.0]])
                e[0] += 1
                for i, (kc, sz) in enumerate(SIZE_COUNTERS.items()):
                    e[1] += c[kc] * sz
                    e[2][i] += c[kc]
        out += ["", "Read requests past L2 by size (no calibration factor), per dispatch:",
                f"{'read_MB':>10} {'req32':>10} {'req64':>10} {'req128':>10}  kernel"]
        tot = 0.0
        for k, (n, by, rq) in sorted(sized.items(), key=lambda kv: -kv[1][1]):
            out.append(f"{by / n / 1e6:10.2f} {rq[0] / n:10.0f} {rq[1] / n:10.0f} "
                       f"{rq[2] / n:10.0f}  {k}")
            tot += by / calls
        out += [f"sized_read_bytes_per_call: {tot:.0f}",
                f"sized_read_over_scaled_fetch: {tot / tot_f:.4f}" if tot_f else ""]
    if len(dirs) == 4:
        cache = {}
        for name, c in _dispatches(dirs[3]):
            if not all(k in c for k in CACHE_COUNTERS):
                continue
            short = _short(name)
            if any(f"sla::{k}<" in name for k in PRODUCT_KERNELS):
                e = cache.setdefault(short, [0.0] * len(CACHE_COUNTERS))
                for i, kc in enumerate(CACHE_COUNTERS):
                    e[i] += c[kc]
        out += ["", "L2 and L1 hit rates (TCC_HIT / (TCC_HIT + TCC_MISS); L1 requests to L2 over",
                "L1 accesses):", f"{'l2_hit':>8} {'l1_to_l2':>9}  kernel"]
        for k, e in sorted(cache.items()):
            l2 = e[0] / max(1.0, e[0] + e[1])
            l1 = e[2] / max(1.0, e[3])
            out.append(f"{l2:8.3f} {l1:9.3f}  {k}")
    print("\n".join(x for x in out if x is not None))


def summarize_counters(args):
    if args.op in ("matvec", "matvec_t", "matvec_vjp"):
        return summarize_product_counters(args)
    p = load_problem(args)
    kernel, kbytes, own, srcs = dominant_kernel(p.method, p.precond, p.n, p.nnz,
                                                p.values.itemsize, p.row_ptr.itemsize,
                                                form_bytes(args.column_form, p))
    names = kernel.split("+")
    dirs = args.summarize_counters
    if len(dirs) not in (2, 3):
        raise SystemExit("--summarize-counters FETCH_DIR WRITE_DIR [SIZES_DIR]")
    f_kib, f_n, f_all, f_pr = _pass_stats(dirs[0], names, "FETCH_SIZE")
    w_kib, w_n, w_all, w_pr = _pass_stats(dirs[1], names, "WRITE_SIZE")
    f_fac = CALIB_BYTES / (f_pr["copy"] * 1024.0)
    w_fac = CALIB_BYTES / (w_pr["copy"] * 1024.0)
    fetch = f_kib * 1024.0 * f_fac
    write = w_kib * 1024.0 * w_fac
    wl = f" --workload {args.workload}"
    out = [
        f"# HBM traffic of {kernel}, workload {p.name}",
        "",
        "Commands (repository root; OUT is any output folder):",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run -- "
        f"python3 bench.py --kernel-only 2{wl}",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run -- "
        f"python3 bench.py --kernel-only 2{wl}",
        "  rocprofv3 --pmc " + " ".join(["TCC_EA0_RDREQ_sum"] + list(SIZE_COUNTERS)) +
        f" --output-format csv -d OUT/pmc_sizes -o run -- python3 bench.py --kernel-only 2{wl}",
        f"  python3 bench.py --summarize-counters OUT/pmc_fetch OUT/pmc_write OUT/pmc_sizes"
        f"{wl}{_form_flag(args)}",
        "",
        "Calibration: the probe kernels of libsla_probe.so in the same run, over 1 GiB:",
        "a copy (reads 1 GiB, writes 1 GiB) and a read-only sum (reads 1 GiB);",
        "factor = 1 GiB / the counter's reading of the copy.",
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
        f"copy_fetch_kib: {f_pr['copy']:.1f}",
        f"copy_write_kib: {w_pr['copy']:.1f}",
    ]
    if "read" in f_pr:
        out.append(f"read_probe_fetch_kib: {f_pr['read']:.1f}")
        out.append(f"read_probe_fetch_factor: {CALIB_BYTES / (f_pr['read'] * 1024.0):.4f}")
    out += [
        f"fetch_factor: {f_fac:.4f}",
        f"write_factor: {w_fac:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"hbm_bytes_per_launch: {fetch + write:.0f}",
        f"algorithmic_bytes_per_launch: {kbytes}",
        f"kernel_bytes_per_launch: {own}",
        f"traffic_over_kernel_bytes: {(fetch + write) / own:.3f}",
    ]
    if len(dirs) == 3:
        by, pr = _size_stats(dirs[2], names)
        out += [
            "",
            "Cross-check from the read-request sizes (32 B x RDREQ_32B + 64 B x RDREQ_64B +",
            "128 B x RDREQ_128B), no calibration factor:",
            f"sized_read_bytes_per_launch: {by:.0f}",
            f"sized_read_over_scaled_fetch: {by / fetch:.4f}",
        ]
        for which in ("copy", "read"):
            if which in pr:
                out.append(f"sized_read_bytes_{which}_probe_over_1GiB: {pr[which] / CALIB_BYTES:.4f}")
    print("\n".join(out))


BLOCK_COUNTERS = ("SQ_INSTS_LDS", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_LDS_STORE_BANDWIDTH",
                  "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CU_CYCLES",
                  "SQ_INSTS_VALU", "SQ_WAIT_INST_LDS")


def summarize_block(args):
    """LDS traffic of the one-workgroup CG solver from one counter run: LDS
    bytes loaded and stored (the BANDWIDTH counters count 64-byte units),
    LDS instructions, bank-conflict and LDS-active cycles, busy compute-unit
    cycles, VALU instructions; per dispatch (forward and adjoint solves
    alternate) and their mean."""
    p = load_problem(args)
    wl = f" --workload {args.workload}" + (" --fp32" if args.fp32 else "")
    rows = [(n, c) for n, c in _dispatches(args.summarize_block) if "sla::block_cg_kernel<" in n]
    if not rows:
        raise SystemExit("no block_cg_kernel dispatches")
    out = [
        f"# LDS counters of block_cg_kernel, workload {p.name}",
        "",
        "Commands (repository root; OUT is any output folder):",
        "  rocprofv3 --pmc " + " ".join(BLOCK_COUNTERS) +
        f" --output-format csv -d OUT/pmc_block -o run -- python3 bench.py --kernel-only 2{wl}",
        f"  python3 bench.py --summarize-block OUT/pmc_block{wl}",
        "",
        f"kernel: {_short(rows[0][0])}",
        f"workload: {p.name}",
        f"n: {p.n}",
        f"batch: {p.batch}",
        f"source_sha256: {sources_sha(['kernels_block.hip', 'sla_internal.h'])}",
        f"dispatches: {len(rows)} (forward and adjoint solves alternate)",
        "",
        f"{'dispatch':>8} {'lds_MB':>10} {'lds_insts':>12} {'bank_confl_cyc':>15} "
        f"{'lds_active_cyc':>15} {'busy_cu_qcyc':>13} {'valu_insts':>12}",
    ]
    tot = {k: 0.0 for k in BLOCK_COUNTERS}
    for i, (_, c) in enumerate(rows):
        lds = (c.get("SQ_INSTS_LDS_LOAD_BANDWIDTH", 0) + c.get("SQ_INSTS_LDS_STORE_BANDWIDTH", 0)) * 64
        out.append(f"{i:8d} {lds / 1e6:10.1f} {c.get('SQ_INSTS_LDS', 0):12.0f} "
                   f"{c.get('SQ_LDS_BANK_CONFLICT', 0):15.0f} {c.get('SQ_LDS_IDX_ACTIVE', 0):15.0f} "
                   f"{c.get('SQ_BUSY_CU_CYCLES', 0):13.0f} {c.get('SQ_INSTS_VALU', 0):12.0f}")
        for k in BLOCK_COUNTERS:
            tot[k] += c.get(k, 0.0)
    m = len(rows)
    lds = (tot["SQ_INSTS_LDS_LOAD_BANDWIDTH"] + tot["SQ_INSTS_LDS_STORE_BANDWIDTH"]) * 64 / m
    out += [
        "",
        f"lds_bytes_per_dispatch: {lds:.0f}",
        f"lds_load_fraction: {tot['SQ_INSTS_LDS_LOAD_BANDWIDTH'] / max(1.0, tot['SQ_INSTS_LDS_LOAD_BANDWIDTH'] + tot['SQ_INSTS_LDS_STORE_BANDWIDTH']):.3f}",
        f"lds_insts_per_dispatch: {tot['SQ_INSTS_LDS'] / m:.0f}",
        f"bank_conflict_over_lds_active: {tot['SQ_LDS_BANK_CONFLICT'] / max(1.0, tot['SQ_LDS_IDX_ACTIVE']):.4f}",
        f"valu_insts_per_lds_inst: {tot['SQ_INSTS_VALU'] / max(1.0, tot['SQ_INSTS_LDS']):.2f}",
        f"lds_wait_quadcycles_per_dispatch: {tot['SQ_WAIT_INST_LDS'] / m:.0f}",
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
        short = _short(name)
        out.append(f"{int(r['Calls']):8d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['TotalDurationNs']) / 1e6:10.2f} {float(r['Percentage']):6.2f}  "
                   f"{short}")
    durs = []
    block = p.method == "cg" and p.n <= 4096
    if block:
        names = ["block_cg_kernel"]  # one launch per solve of the whole batch
        kernel = "block_cg_kernel"
    if args.op != "solve":
        names = []  # the per-kernel block below describes the solve's iteration kernel
    for r in trace:
        if any(f"sla::{s}<" in r["Kernel_Name"] for s in names):
            durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if durs and block:
        out += ["", f"kernel: {kernel}", f"dispatches: {len(durs)}",
                f"avg_us: {sum(durs) / len(durs):.2f}",
                "forward and adjoint solves alternate: " +
                ", ".join(f"{d:.1f}" for d in durs[:8]) + " us"]
    elif durs:
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


# ------------------------------------------------------------------ ceilings

_probe = None


def probe_lib():
    """libsla_probe.so: the streaming and LDS ceiling kernels."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is missing: build it with "
                               "`python -m differentiable_sparse_linear_amd.build`")
        lib = ctypes.CDLL(PROBE_LIB)
        P, I64, D, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int32
        lib.sla_probe_blocks.restype = I32
        lib.sla_probe_read.argtypes = [P, I64, P, P]
        lib.sla_probe_read.restype = I32
        lib.sla_probe_copy.argtypes = [P, P, I64, P]
        lib.sla_probe_copy.restype = I32
        lib.sla_probe_write.argtypes = [P, I64, D, P]
        lib.sla_probe_write.restype = I32
        lib.sla_probe_copy_passes.argtypes = [P, P, I64, I32, P]
        lib.sla_probe_copy_passes.restype = I32
        lib.sla_probe_streams.argtypes = [P, I64, I32, I32, P]
        lib.sla_probe_streams.restype = I32
        lib.sla_probe_lds.argtypes = [I64, P, P]
        lib.sla_probe_lds.restype = I64
        _probe = lib
    return _probe


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def probe_kernels(nbytes, dev, reps=1):
    """Run the probe's read, copy and write kernels over nbytes on the
    current stream, reps times each; returns {name: seconds per call} timed
    with events on that stream (the kernels run there)."""
    import torch
    lib = probe_lib()
    n = nbytes // 8
    a = torch.rand(n, dtype=torch.float64, device=dev)
    b = torch.empty_like(a)
    part = torch.empty(lib.sla_probe_blocks(), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    calls = {"read": lambda: lib.sla_probe_read(_vp(a), n, _vp(part), sp),
             "copy": lambda: lib.sla_probe_copy(_vp(a), _vp(b), n, sp),
             "write": lambda: lib.sla_probe_write(_vp(b), n, 1.0, sp)}
    out = {}
    for name, call in calls.items():
        if call() != 0:  # a first call brings the clocks up
            raise RuntimeError(f"probe {name} failed")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(reps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        out[name] = ev0.elapsed_time(ev1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return out


def measure_ceilings(dev):
    """The chip's bandwidth ceilings in GB/s, measured now: read-only, copy
    (read + write) and write-only over 2 GiB arrays, and LDS reads."""
    import torch
    t = probe_kernels(CEIL_BYTES, dev, reps=10)
    lib = probe_lib()
    part = torch.empty(max(lib.sla_probe_blocks(), 2048), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    lib.sla_probe_lds(100, _vp(part), sp)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    lds_bytes = lib.sla_probe_lds(500, _vp(part), sp)
    ev1.record(stream)
    torch.cuda.synchronize()
    lds_s = ev0.elapsed_time(ev1) * 1e-3
    in_cache = in_cache_copy(dev)
    streams = in_cache_streams(dev)
    return {"read_GBps": CEIL_BYTES / t["read"] / 1e9,
            "copy_GBps": 2 * CEIL_BYTES / t["copy"] / 1e9,
            "write_GBps": CEIL_BYTES / t["write"] / 1e9,
            "lds_GBps": lds_bytes / lds_s / 1e9,
            "arrays_bytes": CEIL_BYTES,
            "copy_GBps_in_cache": in_cache, "in_cache_arrays_bytes": CACHE_CEIL_BYTES,
            "streams_GBps_in_cache": streams, "streams_array_bytes": STREAM_ARRAY_BYTES,
            "kernels": "libsla_probe.so (16 B per access; non-temporal over 2 GiB, plain "
                       "in the cache)"}


STREAM_ARRAY_BYTES = 8_000_000  # one vector of the 1e6-row system
STREAM_SHAPES = ((2, 2), (8, 4), (9, 5), (12, 4))
HBM_STREAM_ARRAY_BYTES = 1 << 30


def in_cache_streams(dev, reps=50, array_bytes=STREAM_ARRAY_BYTES, shapes=STREAM_SHAPES):
    """GB/s of sla_probe_streams, R arrays read and W written per launch, for
    each (R, W) of `shapes`, arrays of `array_bytes` (by default ones that
    stay in the Infinity Cache), one launch per pass as an iteration kernel
    runs: {"RrWw": GB/s}, timed with events over `reps` launches after two."""
    import torch
    lib = probe_lib()
    n = array_bytes // 8
    out = {}
    for r, w in shapes:
        buf = torch.rand((r + w) * n, dtype=torch.float64, device=dev)
        stream = torch.cuda.current_stream()
        sp = ctypes.c_void_p(stream.cuda_stream)
        for _ in range(2):
            if lib.sla_probe_streams(_vp(buf), n, r, w, sp) != 0:
                raise RuntimeError(f"probe streams {r}r{w}w failed")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(reps):
            lib.sla_probe_streams(_vp(buf), n, r, w, sp)
        ev1.record(stream)
        torch.cuda.synchronize()
        sec = ev0.elapsed_time(ev1) * 1e-3 / reps
        out[f"{r}r{w}w"] = (r + w) * array_bytes / sec / 1e9
        del buf
    torch.cuda.empty_cache()
    return out


def in_cache_copy(dev, passes=32, reps=10):
    """Copy bandwidth in GB/s with both arrays (CACHE_CEIL_BYTES each) in the
    Infinity Cache: sla_probe_copy_passes, `passes` ping-pong copies per
    launch, timed with events over `reps` launches after one untimed."""
    import torch
    lib = probe_lib()
    n = CACHE_CEIL_BYTES // 8
    a = torch.rand(n, dtype=torch.float64, device=dev)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    if lib.sla_probe_copy_passes(_vp(a), _vp(b), n, passes, sp) != 0:
        raise RuntimeError("probe copy_passes failed")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(reps):
        lib.sla_probe_copy_passes(_vp(a), _vp(b), n, passes, sp)
    ev1.record(stream)
    torch.cuda.synchronize()
    s = ev0.elapsed_time(ev1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return passes * 2 * CACHE_CEIL_BYTES / s / 1e9


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
    if args.kernel_only:
        for _ in range(args.kernel_only * 10):
            if args.op == "matvec":
                pat.matvec(val, x, out=y)
            elif args.op == "matvec_t":
                pat.matvec(val, g, transpose=True, out=y)
            else:
                pat.matvec_adjoint(val, x, g)
        torch.cuda.synchronize()
        probe_kernels(CALIB_BYTES, dev)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only, "calls": args.kernel_only * 10,
                          "calibration_bytes": CALIB_BYTES}))
        return
    # a pattern with rows past the tile walker's slots (the graph) also runs
    # the row plan's kernels
    plan = "+plan_spmv_kernel+plan_finish_kernel" if args.graph else ""
    if args.op == "matvec":
        call = lambda: pat.matvec(val, x, out=y)
        # values + columns + row pointers, x once, y written
        model = p.nnz * (sv + 4) + (p.n + 1) * sr + 2 * p.n * sv
        kernel = "spmv_kernel" + plan
    elif args.op == "matvec_t":
        call = lambda: pat.matvec(val, g, transpose=True, out=y)
        model = product_model_bytes(args.op, p) // p.batch
        # with diagonal masks one kernel reads A's own rows; else the terms
        # pass over A's rows and the row sums of A^T
        kernel = ("diag_vjp_kernel" if pat.column_mode() == "diagonal"
                  else "grad_kernel+rowsum_kernel" + ("+plan_grad_kernel" if plan else "") + plan)
    else:
        call = lambda: pat.matvec_adjoint(val, x, g)
        # values + columns + row pointers once, g, x read, grad_x and
        # grad_values written
        model = p.nnz * (2 * sv + 4) + (p.n + 1) * sr + 3 * p.n * sv
        # with diagonal masks one kernel makes both from A's own rows; else a
        # pass over A's rows writes grad_values and scatters the terms of
        # A^T g to A^T's order, and a second pass sums A^T's rows
        kernel = ("diag_vjp_kernel" if pat.column_mode() == "diagonal"
                  else "grad_kernel+rowsum_kernel" + ("+plan_grad_kernel" if plan else "") + plan)
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
    traffic = read_product_traffic(
        args.op, p.name, sources_sha(["kernels_spmv.hip", "spmv_tile.h", "sla_internal.h"]))
    dram = traffic / per / 1e9 if traffic else None
    print(json.dumps({
        "metric": f"differentiable {args.op} calls/sec", "value": steps / wall,
        "unit": "calls/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": wall * 1e3 / steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64" if p.values.dtype == np.float64 else "f32",
        "data": "synthetic", "config": {"workload": p.name, "n": p.n, "nnz": p.nnz,
                                        "batch": p.batch},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "dram_GBps": dram,
                     "dram_frac": dram / HBM_PEAK_GBPS if dram else None,
                     "bytes_per_launch": model, "avg_launch_us": per * 1e6},
    }), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_block:
        return summarize_block(args)
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
    if args.graph and args.op not in ("matvec", "matvec_t", "matvec_vjp"):
        print("--graph is for --op matvec / matvec_t / matvec_vjp", file=sys.stderr)
        sys.exit(2)
    if args.op == "inverse":
        return bench_inverse(args)
    p = load_problem(args)
    print(f"workload {p.name} ready", file=sys.stderr, flush=True)
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
        for i in range(args.kernel_only):
            step()
            torch.cuda.synchronize()
            print(f"kernel-only: step {i + 1} of {args.kernel_only} done", file=sys.stderr,
                  flush=True)
        # known-traffic kernels for the counters' calibration: copy, read, write of 1 GiB
        probe_kernels(CALIB_BYTES, dev)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only, "calibration_bytes": CALIB_BYTES}))
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
    ceilings = measure_ceilings(dev)
    # a working set beyond the Infinity Cache (the 512^3 system's): the same
    # stream launches over arrays of 1 GiB, read from and written to HBM
    big = p.n * 13 * p.values.itemsize > (256 << 20)
    if big:
        ceilings["streams_GBps_hbm"] = in_cache_streams(
            dev, reps=5, array_bytes=HBM_STREAM_ARRAY_BYTES, shapes=((8, 4), (9, 5)))
        ceilings["streams_hbm_array_bytes"] = HBM_STREAM_ARRAY_BYTES
    if block_path:
        roofline = block_roofline(p, pat, val, b, x, opts, stream)
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
        traffic = read_traffic(kernel, p.name, sources_sha(srcs))
        dram = traffic / k_avg_s / 1e9 if traffic else None
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": traffic,
                    "model_frac": achieved / HBM_PEAK_GBPS,
                    "bytes_per_launch": kbytes, "kernel_bytes_per_launch": own,
                    "iteration_form": form, "kernel_GBps": own / k_avg_s / 1e9,
                    "kernel_frac": own / k_avg_s / 1e9 / HBM_PEAK_GBPS,
                    "dram_GBps": dram, "dram_frac": dram / HBM_PEAK_GBPS if dram else None,
                    "dram_frac_of_copy_ceiling": dram / ceilings["copy_GBps"] if dram else None,
                    # a working set within the Infinity Cache (the 1e6-row
                    # 3D diffusion system's) is read past L2 from the cache
                    # and written into it: this is its ceiling
                    "dram_frac_of_in_cache_copy_ceiling":
                        dram / ceilings["copy_GBps_in_cache"] if dram else None,
                    # the same against pure streams of the CG iteration's
                    # shape in the cache (8 vectors read and 4 written on
                    # even launches, 9 and 5 on odd ones), one launch each
                    "dram_frac_of_in_cache_stream_ceiling":
                        dram / (0.5 * (ceilings["streams_GBps_in_cache"]["8r4w"] +
                                       ceilings["streams_GBps_in_cache"]["9r5w"]))
                        if dram else None,
                    # beyond the cache: against the same launches over 1 GiB arrays
                    "dram_frac_of_hbm_stream_ceiling":
                        dram / (0.5 * (ceilings["streams_GBps_hbm"]["8r4w"] +
                                       ceilings["streams_GBps_hbm"]["9r5w"]))
                        if dram and "streams_GBps_hbm" in ceilings else None,
                    "avg_launch_us": k_avg_s * 1e6, "launches_timed": k_n,
                    "hbm_target": "at least 70 % of peak HBM bandwidth, read as dram_frac "
                                  "(bytes past L2 by the counters; model_frac prices a launch at "
                                  "the textbook iteration's bytes, kernel_frac at the fused "
                                  "kernel's own)"}
    memory = peak_memory(pat, step)

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
        "ceilings": ceilings,
        "memory": memory,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(result), flush=True)


def block_roofline(p, pat, val, b, x, opts, stream):
    """The one-workgroup CG solver keeps p and x in LDS (p is gathered by
    every row's product) and r, M^-1, the row's own p and the matrix in
    registers, so its bound is LDS bandwidth.  Per row and iteration it
    gathers S entries of p (S slots: the longest row), stores the new p and
    reads and writes x: S + 3 values; with fp64 and four rows per thread
    M^-1 is read from LDS twice more (S + 5), and without the resident
    matrix r and the own p as well (S + 11).  One forward solve is timed
    with events on the stream it runs on; the peak is the LDS of the compute
    units the batch occupies (one workgroup of 1024 threads per unit)."""
    import torch
    sv = p.values.itemsize
    rows = np.diff(p.row_ptr)
    longest = int(rows.max())
    S = 4 if longest <= 4 else (longest if longest in (5, 6) else 8)
    rpt = (p.n + 1023) // 1024
    resident = longest <= 8 and rpt * (S * (sv // 4) + (S + 1) // 2) <= 56
    dreg = sv == 4 or rpt <= 2
    per_row = (S + 3 + (0 if dreg else 2) + (0 if dreg or resident else 6)) * sv
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    _, fi = pat.solve(val, b, out=x, **opts)
    ev1.record(stream)
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) * 1e-3
    lds = int(fi["iters"].astype(np.int64).sum()) * p.n * per_row
    cus = min(p.batch, 256)
    peak = LDS_PEAK_CU_GBPS * cus
    achieved = lds / t / 1e9
    return {"bound": "lds", "kernel": "block_cg_kernel", "achieved": achieved, "peak": peak,
            "unit": "GB/s", "frac": achieved / peak, "traffic": None,
            "lds_bytes_per_row_iteration": per_row, "slots": S,
            "forward_ms": t * 1e3, "compute_units": cus,
            "system_iterations_per_s": float(fi["iters"].sum()) / t}


def peak_memory(pat, step):
    """Device memory of one forward + adjoint step: the handle's workspace
    (allocated once at create) and the peak of the caller's tensors (values,
    b, x, the gradients) that torch holds, beside the pages' figures for
    context (naive backpropagation through 1000 CG iterations at 1e6 unknowns
    estimated at about 80 GB; the adjoint measured at about 328 MB, 195 times
    less; Problem statement and Results of the torch-sla explainer)."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    peak = int(torch.cuda.max_memory_allocated())
    ws = int(pat.workspace_bytes())
    return {"handle_workspace_bytes": ws, "torch_peak_bytes": peak,
            "peak_device_bytes": ws + peak,
            "pages_context": {"naive_backprop_GB_estimate": 80, "adjoint_MB_measured": 328,
                              "reduction": 195}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(p, budget_s, maxit):
    """Forward + adjoint oracle solves of the batch's systems in order, each
    cut to `maxit` iterations each way, until about budget_s seconds have
    passed (at least one system): (iterations, systems, seconds)."""
    import oracle as O
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
    return its, systems, time.perf_counter() - t0


def cpu_baseline(p, budget_s=15.0, serial_budget_s=8.0):
    """The oracle (plain fp64 C, OpenMP loops, fixed-order dot products) on
    bounded samples of the same workload, on this host's cores: whole
    forward + adjoint solves on all threads for about budget_s seconds
    (systems whose solve would take many minutes, n * maxit > 1e10, the
    512^3 case, cut to 5 iterations each way), then the same on one thread
    (set in-process), cut to as many iterations each way as fit about
    serial_budget_s seconds.  Rates in iterations (summed over systems) per
    second."""
    import oracle as O
    maxit = 5 if p.n * p.maxit > 1e10 else p.maxit
    threads = O.num_threads()
    its, systems, t = _oracle_rate(p, budget_s, maxit)
    cut = f", cut to {maxit} iterations each way" if maxit != p.maxit else ""
    rate = its / t
    # one thread: iterations per second are at best the all-thread rate over
    # the threads; size the cut from it
    O.set_num_threads(1)
    try:
        per_it = threads / rate
        m1 = int(max(2, min(maxit, serial_budget_s / (2 * per_it))))
        its1, sys1, t1 = _oracle_rate(p, serial_budget_s, m1)
    finally:
        O.set_num_threads(threads)
    return {"value": rate, "unit": "PCG iterations/s", "cores": threads, "kind": "oracle",
            "sample": f"forward + adjoint solves of {systems} of {p.batch} system(s) of {p.name}"
                      f"{cut} ({its} iterations, {t:.1f} s)",
            "single_core": {"value": its1 / t1, "unit": "PCG iterations/s", "cores": 1,
                            "sample": f"forward + adjoint solves of {sys1} system(s) cut to "
                                      f"{m1} iterations each way ({its1} iterations, "
                                      f"{t1:.1f} s)"},
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}


if __name__ == "__main__":
    main()
