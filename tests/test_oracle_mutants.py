"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of ``oracle/oracle.c`` with one plausible slip (a
dropped log-weight, a flipped sign, a missing 1/eps, a halved cost, the wrong
marginal, an unstabilised sum, a missing a_i in the plan, a wrong annealing
exponent), compiled on the CPU into a temporary library.  The fast pins of
``test_oracle_pins.py`` are then run against it; at least one must fail.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_log_weight": ("z[k] = (pot[k] - c) / eps + log(w[k]);", "z[k] = (pot[k] - c) / eps;"),
    "flip_potential_sign": ("z[k] = (pot[k] - c) / eps", "z[k] = (-pot[k] - c) / eps"),
    "missing_inverse_eps": ("z[k] = (pot[k] - c) / eps", "z[k] = (pot[k] - c)"),
    "half_cost": ("c += u * u;", "c += 0.5 * u * u;"),
    "wrong_weights_in_g_update": ("if (oracle_g_update(X, Y, a, f, n, m, d, eps, g)) return 1;",
                                  "if (oracle_g_update(X, Y, b, f, n, m, d, eps, g)) return 1;"),
    "unstabilised_sum": ("s += exp(z[k] - zmax);", "s += exp(z[k]);"),
    "plan_without_a": ("if (!divide_by_a) p *= a[i];", ""),
    "wrong_residual_marginal": ("rsum += fabs(s - a[i]);", "rsum += fabs(s - b[i]);"),
    "wrong_anneal_exponent": ("(double)s / (double)(n_stages - 1)", "(double)s / (double)n_stages"),
    "skip_first_f_update": ("if (oracle_f_update(X, Y, b, g, n, m, d, eps, f)) return 1;",
                                      "if (it > 0 && oracle_f_update(X, Y, b, g, n, m, d, eps, f)) return 1;"),
}


FAST_PINS = [
    lambda: pins.test_p1_scaling_form_iterate_for_iterate(0, 20, 20, 3, 0.3),
    lambda: pins.test_p1_scaling_form_iterate_for_iterate(1, 31, 31, 5, 0.1),
    pins.test_p5_single_target_point,
    pins.test_p5_coincident_clouds,
    pins.test_p5_two_point_closed_form,
    lambda: pins.test_p4_softmin_brackets_every_f_update(30),
    lambda: pins.test_p6_p7_marginals_and_dual_ascent(50),
    pins.test_p10_power_of_two_scaling_bit_exact,
    pins.test_annealing_schedule_end_points,
]


def _square_residual_transport_pin():
    X, Y, a, b = pins.small_problem(120, 19, 19, 3)
    rng = np.random.default_rng(121)
    f = rng.standard_normal(19) * 0.1
    g = rng.standard_normal(19) * 0.1
    V = rng.standard_normal((19, 5))
    eps = 0.4
    P = pins.dense_plan(X, Y, a, b, f, g, eps)
    _, rt, ct = oracle.marginal_residual(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(rt, np.abs(P.sum(1) - a).sum(), rtol=1e-12)
    np.testing.assert_allclose(ct, np.abs(P.sum(0) - b).sum(), rtol=1e-12)
    np.testing.assert_allclose(oracle.transport(X, Y, a, b, f, g, V, eps), P @ V, rtol=1e-12)


def _square_sinkhorn_pin():
    X, Y, a, b = pins.small_problem(7, 24, 24, 3)
    C = pins.dense_cost(X, Y)
    eps = 0.3 * np.median(C)
    K = np.exp(-C / eps)
    v = b.copy()
    for _ in range(5):
        u = a / (K @ v)
        v = b / (K.T @ u)
    res = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=5)
    np.testing.assert_allclose(res["f"], eps * np.log(u / a), rtol=1e-10)
    np.testing.assert_allclose(res["g"], eps * np.log(v / b), rtol=1e-10)


FAST_PINS += [_square_residual_transport_pin, _square_sinkhorn_pin]
# Pins whose problems have n == m: the only ones run against mutants that
# swap an n-vector for an m-vector (otherwise the mutant would read past an
# array on the CPU).
SQUARE_PINS = FAST_PINS[:2] + [_square_residual_transport_pin, _square_sinkhorn_pin]
LENGTH_SWAPPING = {"wrong_weights_in_g_update", "wrong_residual_marginal"}


def test_unmutated_source_passes_fast_pins():
    for pin in FAST_PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", str(c_path),
                    "-o", str(so_path), "-lm"], check=True)
    monkeypatch.setattr(oracle, "LIB_PATH", str(so_path))
    monkeypatch.setattr(oracle, "_lib", None)
    caught = []
    for pin in (SQUARE_PINS if name in LENGTH_SWAPPING else FAST_PINS):
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught.append(pin)
    monkeypatch.setattr(oracle, "_lib", None)
    assert caught, f"mutant {name} survived every pin"
