"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them.  This is evidence that the pins constrain
each part of the oracle: coefficient, key norm, forcing term, sign, readout,
layout and initial state.
"""
import contextlib
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "efla_oracle.c")

MUTATIONS = {
    "euler_coefficient": ("return beta * (-expm1(-x) / x);", "return beta;"),
    "coefficient_sign": ("return beta * (-expm1(-x) / x);", "return beta * (expm1(x) / x);"),
    "norm_not_squared": ("lam += k[i] * k[i];\n    const double a", "lam += fabs(k[i]);\n    const double a"),
    "dropped_forcing": ("+= -a * k[i] * kS[j] + a * k[i] * v[j];", "+= -a * k[i] * kS[j];"),
    "flipped_decay_sign": ("+= -a * k[i] * kS[j] + a * k[i] * v[j];", "+= a * k[i] * kS[j] + a * k[i] * v[j];"),
    "wrong_projection_operand": ("acc += k[i] * S[(int64_t)i * dv + j];", "acc += q[i] * S[(int64_t)i * dv + j];"),
    "readout_uses_key": ("acc += S[(int64_t)i * dv + j] * q[i];", "acc += S[(int64_t)i * dv + j] * k[i];"),
    "swapped_batch_head_layout": ("const int64_t row = (b * J->L + t) * J->H + h;",
                                  "const int64_t row = (h * J->L + t) * J->B + b;"),
    "rule_ignored": ("return rule == 1 ? beta : oracle_alpha(beta, lam);",
                     "return oracle_alpha(beta, lam);"),
    "rules_swapped": ("return rule == 1 ? beta : oracle_alpha(beta, lam);",
                      "return rule == 0 ? beta : oracle_alpha(beta, lam);"),
    "euler_half_step": ("return rule == 1 ? beta : oracle_alpha(beta, lam);",
                        "return rule == 1 ? 0.5 * beta : oracle_alpha(beta, lam);"),
    "forward_drops_rule": ("B, H, dk, dv, L, nthreads, i, rule};", "B, H, dk, dv, L, nthreads, i, 0};"),
    "bwd_dq_reads_previous_state": ("acc += St[(int64_t)i * dv + j] * dO[j];", "acc += Sp[(int64_t)i * dv + j] * dO[j];"),
    "bwd_state_grad_misses_projection": ("dS[(int64_t)i * dv + j] -= k[i] * du[j];",
                                         "dS[(int64_t)i * dv + j] -= 0.0 * k[i] * du[j];"),
    "bwd_psi_series_sign": ("        return -sum;", "        return sum;"),
    "bwd_dbeta_of_euler_in_exact": ("    *da_db = exp(-x);", "    *da_db = 1.0;"),
    "bwd_dk_drops_lambda_term": ("dkk[i] = a * acc1 - acc2 + 2.0 * dlam * k[i];", "dkk[i] = a * acc1 - acc2;"),
    "bwd_du_unscaled": ("du[j] = a * acc;", "du[j] = acc;"),
    "initial_state_ignored": ("memcpy(S, J->s0 + u * sdim, sizeof(double) * (size_t)sdim);",
                              "memset(S, 0, sizeof(double) * (size_t)sdim);"),
}

PINS = [
    lambda: pins.test_alpha_matches_60_digit_evaluation(0.5),
    pins.test_alpha_limits,
    pins.test_coeff_lambda_is_squared_norm,
    lambda: pins.test_P1_closed_form_matches_taylor_expm(12, 4.0, 1.1),
    lambda: pins.test_P2_exact_step_matches_rk4(22, 4.0, 0.9),
    pins.test_P2b_forward_matches_ode_solution_all_heads,
    pins.test_P3_P5_projection_invariants,
    pins.test_P4_euler_limit,
    pins.test_P6_stiff_limit_overwrites,
    pins.test_P9_scalar_closed_form,
    pins.test_forward_threads_and_layout,
    pins.test_P11_euler_coefficient_is_beta,
    pins.test_P11_euler_projection_invariants,
    pins.test_P11_euler_unit_step_overwrites_and_large_step_expands,
    pins.test_P11_euler_orthonormal_keys_store_values,
    pins.test_P11_euler_forward_equals_euler_steps_and_limits,
    lambda: pins.test_P12_backward_matches_finite_differences("exact", "moderate"),
    lambda: pins.test_P12_backward_matches_finite_differences("exact", "stiff"),
    lambda: pins.test_P12_backward_matches_finite_differences("euler", "moderate"),
    lambda: [pins.test_P12_alpha_derivatives_against_60_digit_differentiation(x, 1.0) for x in (1e-3, 0.3)],
]


@contextlib.contextmanager
def _swapped_lib(path):
    saved_lib, saved_path = oracle._lib, oracle._LIB_PATH
    oracle._lib, oracle._LIB_PATH = None, path
    try:
        oracle._load()
        yield
    finally:
        oracle._lib, oracle._LIB_PATH = saved_lib, saved_path


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
                    "-pthread", str(mutated), "-o", str(lib), "-lm"], check=True)
    failed = []
    with _swapped_lib(str(lib)):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin)
    assert failed, f"no pin caught the planted mistake '{name}'"


def test_unmutated_oracle_passes_all_pins():
    for pin in PINS:
        pin()
    assert isinstance(oracle._load(), ctypes.CDLL)
