"""Pins of the oracle's Hessian-vector product (oracle/hvp.py).

The pages give no formula for the HVP; the oracle's is a derivation (implicit
differentiation through the fixed point, see its header).  Pinned by what the
derivation does not use:

H1  central finite differences of the gradient at potentials re-converged at
    X + hV and X - hV (the gradient itself pinned by finite differences of
    the converged loss in test_oracle_gradient.py);
H2  symmetry <U, H V> = <V, H U> at converged potentials;
H3  a single target point: P_i1 = a_i whatever X is, so the gradient is
    2 a_i (x_i - y_1) and H V = 2 a V exactly.
A planted slip (a dropped potential derivative, a dropped diagonal term) is
caught by H1.
"""
import numpy as np
import pytest

import oracle
from oracle.hvp import hvp


def _problem(seed, n, m, d):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d)) * 0.8
    Y = rng.standard_normal((m, d)) * 0.6 + 0.3
    a = rng.standard_exponential(n)
    b = rng.standard_exponential(m)
    return X, Y, a / a.sum(), b / b.sum()


def _converged(X, Y, a, b, eps):
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=20000, tol=1e-14, check_every=10)
    assert r["residual"] <= 1e-12
    return r["f"], r["g"]


def _grad(X, Y, a, b, eps):
    f, g = _converged(X, Y, a, b, eps)
    return oracle.gradient(X, Y, a, b, f, g, eps)[0]


@pytest.mark.parametrize("seed,n,m,d,eps", [(1, 6, 5, 2, 0.5), (2, 5, 7, 3, 0.3)])
def test_h1_finite_differences_of_the_gradient(seed, n, m, d, eps):
    X, Y, a, b = _problem(seed, n, m, d)
    V = np.random.default_rng(seed + 10).standard_normal((n, d))
    f, g = _converged(X, Y, a, b, eps)
    H = hvp(X, Y, a, b, f, g, V, eps)
    h = 1e-5
    fd = (_grad(X + h * V, Y, a, b, eps) - _grad(X - h * V, Y, a, b, eps)) / (2 * h)
    assert np.max(np.abs(fd - H)) <= 1e-6 * (1 + np.max(np.abs(H))), np.max(np.abs(fd - H))


def test_h2_symmetry():
    X, Y, a, b = _problem(3, 7, 6, 3)
    eps = 0.4
    f, g = _converged(X, Y, a, b, eps)
    rng = np.random.default_rng(4)
    U, V = rng.standard_normal((7, 3)), rng.standard_normal((7, 3))
    lhs = np.sum(U * hvp(X, Y, a, b, f, g, V, eps))
    rhs = np.sum(V * hvp(X, Y, a, b, f, g, U, eps))
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + abs(rhs))


def test_h3_single_target():
    X, Y, a, b = _problem(5, 8, 1, 3)
    eps = 0.3
    f, g = _converged(X, Y, a, b, eps)
    V = np.random.default_rng(6).standard_normal((8, 3))
    np.testing.assert_allclose(hvp(X, Y, a, b, f, g, V, eps), 2 * a[:, None] * V,
                               rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mutant", ["no_potential_terms", "no_diagonal"])
def test_h1_catches_planted_slips(mutant):
    # The slip is planted in a copy of the oracle's arithmetic on the CPU.
    X, Y, a, b = _problem(1, 6, 5, 2)
    eps = 0.5
    V = np.random.default_rng(11).standard_normal((6, 2))
    f, g = _converged(X, Y, a, b, eps)
    H, parts = hvp(X, Y, a, b, f, g, V, eps, return_parts=True)
    from oracle.hvp import plan
    P = plan(X, Y, a, b, f, g, eps)
    D = X[:, None, :] - Y[None, :, :]
    dC = 2.0 * np.einsum("ijk,ik->ij", D, V)
    if mutant == "no_potential_terms":
        bad = 2 * parts["r"][:, None] * V + 2 * np.einsum("ij,ijk->ik", -P * dC / eps, D)
    else:
        dP = P * (parts["df"][:, None] + parts["dg"][None, :] - dC) / eps
        bad = 2 * np.einsum("ij,ijk->ik", dP, D)
    h = 1e-5
    fd = (_grad(X + h * V, Y, a, b, eps) - _grad(X - h * V, Y, a, b, eps)) / (2 * h)
    assert np.max(np.abs(fd - H)) <= 1e-6 * (1 + np.max(np.abs(H)))
    assert np.max(np.abs(fd - bad)) > 1e-3 * (1 + np.max(np.abs(H)))
