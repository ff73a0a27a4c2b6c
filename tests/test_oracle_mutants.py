"""The pins must reject plausible mistakes in the oracle.

Each case copies oracle.c, plants one mistake (a dropped term, a wrong sign, a
transposed operand, a wrong index), builds it with gcc into a temporary
directory and runs every pin against it.  At least one pin has to fail.
Everything here runs on the CPU.
"""
import os

import pytest

import oracle as O
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")

MUTANTS = {
    "grad_sign": ("grad_val[k] = -(lam[i] * x[col[k]]);", "grad_val[k] = (lam[i] * x[col[k]]);"),
    "grad_transposed": ("grad_val[k] = -(lam[i] * x[col[k]]);", "grad_val[k] = -(x[i] * lam[col[k]]);"),
    "adjoint_uses_A": ("vt[k] = val[perm[k]];", "vt[k] = val[k];"),
    "spmv_index": ("s += val[k] * x[col[k]];", "s += val[k] * x[i];"),
    "cg_beta_inverted": ("double beta = rho_new / rho;", "double beta = rho / rho_new;"),
    "cg_no_precond": ("z[i] = precond ? dinv[i] * r[i] : r[i];", "z[i] = r[i];"),
    "cg_r_update_sign": ("r[i] -= alpha * q[i];", "r[i] += alpha * q[i];"),
    "bicg_p_sign": ("p[i] = r[i] + beta * (p[i] - omega * v[i]);",
                    "p[i] = r[i] + beta * (p[i] + omega * v[i]);"),
    "bicg_x_drops_omega_s": ("x[i] += alpha * p[i] + omega * s[i];", "x[i] += alpha * p[i];"),
    "bicg_half_step_skips_x": ("                x[i] += alpha * p[i];\n            rnorm = snorm;",
                               "                x[i] += 0.0 * p[i];\n            rnorm = snorm;"),
    "vjp_grad_x_not_transposed": ("grad_x[col[k]] += val[k] * gy[i];",
                                  "grad_x[i] += val[k] * gy[col[k]];"),
    "vjp_grad_val_transposed": ("grad_val[k] = gy[i] * x[col[k]];",
                                "grad_val[k] = x[i] * gy[col[k]];"),
    "bicg_nan_denominator_passes": ("if (!(fabs(tt) > 0.0) || !(fabs(ts) > 0.0)) {",
                                    "if (tt == 0.0 || ts == 0.0) {"),
    "transpose_unstable": ("int64_t dst = next[col[k]]++;", "int64_t dst = next[col[k]]; next[col[k]] += 1; dst = row_ptr_t[col[k] + 1] - 1 - (dst - row_ptr_t[col[k]]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mut = src.replace(old, new)
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(mut)
    lib = O.compile_source(str(path), str(tmp_path / f"lib_{name}.so"))
    failed = []
    with O.using_library(lib):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
            except Exception as e:  # a crash or numeric blow-up also counts as caught
                failed.append(f"{pin.__name__}:{type(e).__name__}")
    assert failed, f"no pin caught mutant {name}"
