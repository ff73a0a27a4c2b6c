"""C-ABI checks that need no GPU: the library builds, loads, and exports every
function ``include/sla.h`` declares.  No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def libpath():
    import differentiable_sparse_linear_amd as sla
    if not os.path.exists(sla.LIB_PATH):
        from differentiable_sparse_linear_amd import build
        build.build()
    return sla.LIB_PATH


def test_header_declares_the_boundary():
    names = _declared()
    for f in ("sla_create", "sla_destroy", "sla_matvec", "sla_solve", "sla_solve_adjoint"):
        assert f in names


def test_library_exports_every_declared_symbol(libpath):
    lib = ctypes.CDLL(libpath)
    missing = [f for f in _declared() if not hasattr(lib, f)]
    assert not missing, missing
    import differentiable_sparse_linear_amd as sla
    assert set(_declared()) == set(sla.EXPORTED_SYMBOLS)


def test_probe_library_exports_its_header():
    """The benchmark's ceiling kernels (libsla_probe.so) export every
    function include/sla_probe.h declares."""
    import differentiable_sparse_linear_amd.build as b
    if not os.path.exists(b.PROBE_LIB):
        b.build_probe()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "sla_probe.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(sla_probe_[a-z_]+)\s*\(", text)))
    assert names == ["sla_probe_blocks", "sla_probe_copy", "sla_probe_copy_passes",
                     "sla_probe_lds", "sla_probe_read", "sla_probe_streams", "sla_probe_write"]
    lib = ctypes.CDLL(b.PROBE_LIB)
    assert all(hasattr(lib, f) for f in names)
    # argument checks return before any launch
    assert lib.sla_probe_read(None, 8, None, None) == -1
    assert lib.sla_probe_copy(None, None, 8, None) == -1
    assert lib.sla_probe_streams(None, ctypes.c_int64(8), 2, 2, None) == -1


def test_status_strings_and_null_handle(libpath):
    import differentiable_sparse_linear_amd as sla
    lib = sla.load(libpath)
    for st in (0, 1, 2, -1, -2, -3, -4, -5, -6):
        assert lib.sla_status_string(st)
    assert b"unknown" not in lib.sla_status_string(-6)
    # pure argument checks return before touching the device
    assert lib.sla_destroy(None) == sla.SLA_ERR_ARG
    assert lib.sla_workspace_bytes(None) == -1
    assert lib.sla_create(None, 4, 4, 1, 1, 0, None, None, 0, None) == sla.SLA_ERR_ARG
    h = ctypes.c_void_p()
    assert lib.sla_create(ctypes.byref(h), 0, 4, 1, 1, 0, None, None, 0, None) == sla.SLA_ERR_ARG
    assert lib.sla_solve(None, None, None, None, None, None, None) == sla.SLA_ERR_ARG
    assert lib.sla_matvec_adjoint(None, None, None, None, None, None, None) == sla.SLA_ERR_ARG
    # the no-alloc solve: sizes beyond its fixed scratch, and missing pointers
    p = ctypes.c_void_p(16)
    na = lib.sla_solve_noalloc
    assert na(4097, 4097, 1, 1, 0, p, p, p, p, p, None, None, None) == sla.SLA_ERR_TOO_LARGE
    assert na(64, 64, 65536, 1, 0, p, p, p, p, p, None, None, None) == sla.SLA_ERR_TOO_LARGE
    assert na(64, 64, 1, 1, 0, None, p, p, p, p, None, None, None) == sla.SLA_ERR_ARG
    assert na(64, 63, 1, 1, 0, p, p, p, p, p, None, None, None) == sla.SLA_ERR_ARG
    assert na(64, 64, 1, 2, 0, p, p, p, p, p, None, None, None) == sla.SLA_ERR_ARG
    bicg = sla._make_opts(1e-10, 10, "bicgstab", "none", 0, 0, 0)
    assert na(64, 64, 1, 1, 0, p, p, p, p, p, ctypes.byref(bicg), None, None) == sla.SLA_ERR_ARG


def test_product_path_has_no_oracle_or_fallback():
    pkg = os.path.join(ROOT, "differentiable_sparse_linear_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f


def test_bench_modes_parse_and_refuse_more_gpus():
    """bench.py: every --op parses, and --gpus above 1 exits with a message
    before touching a GPU (host check)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for op in ("solve", "matvec", "matvec_t", "matvec_vjp", "inverse", "nonlinear", "eigsh"):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--op", op,
                            "--gpus", "2"], capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and "one GPU" in r.stderr, (op, r.stderr)


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes mirrors of sla_solve_opts, sla_solve_info and sla_eig_opts
    have the C structs' sizes and member offsets (a plain C program built
    with gcc against include/sla.h prints them)."""
    import shutil
    import subprocess
    import differentiable_sparse_linear_amd as sla
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    structs = {"sla_solve_opts": sla._Opts, "sla_solve_info": sla._Info,
               "sla_eig_opts": sla._EigOpts}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "sla.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True,
                             text=True).stdout.splitlines():
        cname, member, v = ln.split()
        got[(cname, member)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_bench_bytes_model():
    """The bench's per-launch byte counts for the 1e6-DOF workload: the
    textbook PCG iteration (CSR with int32 columns, SpMV plus 11 vector
    passes) and the fused kernel's own bytes in each storage form."""
    import numpy as np
    import bench
    import workloads as W
    n, nnz = 1_000_000, 6_940_000
    k, alg, own, _ = bench.dominant_kernel("cg", "jacobi", n, nnz, 8, 4, 7 * n * 8)
    assert k == "cg_iter_kernel"
    assert alg == nnz * 12 + (n + 1) * 4 + 13 * n * 8 == 191_280_004
    assert own == 7 * n * 8 + 9 * n * 8
    p = W.config(2, size=12)
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    assert np.unique(p.col - rows).size == 7
    assert bench.form_bytes("diagonal-major", p) == 7 * p.n * 8
    assert bench.form_bytes("diagonal-major-symmetric", p) == 4 * p.n * 8
    assert bench.form_bytes("diagonal", p) == p.nnz * 8 + 2 * p.n + (p.n + 1) * 4
    assert bench.form_bytes("wide", p) == p.nnz * 12 + (p.n + 1) * 4
