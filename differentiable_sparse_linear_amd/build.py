"""Build libsla.so (every HIP source under csrc/) and the benchmark's
bandwidth-ceiling kernels libsla_probe.so (probe/) for gfx950 with hipcc.

    python -m differentiable_sparse_linear_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsla.so")
PROBE_SRC = os.path.join(PKG, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "libsla_probe.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from forming packed FP32 arithmetic.
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, out: str = LIB, defines=(), tmpdir: str = None) -> str:
    """Compile every csrc/*.hip and link ``out``; ``defines`` are extra -D flags."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    tmpdir = tmpdir or os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    procs = []
    for src in sources():
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *[f for f in FLAGS if f != "-shared"], *[f"-D{d}" for d in defines], "-c",
               "-I", INCLUDE, "-I", CSRC, src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd)))
        objs.append(obj)
    failed = [src for src, p in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False, out: str = PROBE_LIB) -> str:
    """Compile and link the bandwidth-ceiling kernels."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc, *FLAGS, "-I", INCLUDE, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
