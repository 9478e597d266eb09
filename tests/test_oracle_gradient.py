"""Pins of the oracle's gradient, dual objective and column-side transport.

The explainer ("Method" part 3) states that gradients with respect to the
points, like the barycentric projection, are weighted averages under the
plan; it prints no formula or value.  The oracle writes the gradient of the
dual objective
    D(f, g; X, Y) = <a,f> + <b,g> - eps sum_ij a_i b_j (exp((f_i+g_j-C_ij)/eps) - 1)
at fixed potentials as grad_x_i = 2 sum_j P_ij (x_i - y_j) (and the mirror
for y).  Pinned here by what it does not compute itself:

G1  central finite differences of the entropic OT value (the dual at the
    converged potentials, re-solved at every perturbed point): the envelope
    theorem makes its derivative the gradient at the optimum;
G2  central finite differences of D at fixed, unconverged potentials (a
    different oracle function, summing the exponential terms pair by pair);
G3  translation invariance: sum_i grad_x_i + sum_j grad_y_j = 0 at any (f, g);
G4  a single target point: at convergence P_i1 = a_i, so
    grad_x_i = 2 a_i (x_i - y_1);
G5  the dual objective equals <a,f> + <b,g> after an f- or g-update (equal
    total masses), and lies in the brute-force assignment brackets
    W <= D <= W + eps log n at convergence;
G6  the column-side transport is the transpose of the row-side one against a
    dense plan.
Each catches a plausible slip: a missing factor 2, a sign, a swapped weight,
a transposed plan.
"""
import itertools

import numpy as np
import pytest

import oracle


def _problem(seed, n, m, d, offset=0.4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d)) * 0.7 + offset
    a = rng.standard_exponential(n)
    b = rng.standard_exponential(m)
    return X, Y, a / a.sum(), b / b.sum()


def _converged(X, Y, a, b, eps):
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=20000, tol=1e-13, check_every=10)
    assert r["residual"] <= 1e-12
    return r["f"], r["g"]


def _ot_value(X, Y, a, b, eps):
    f, g = _converged(X, Y, a, b, eps)
    return float(a @ f + b @ g)


def test_g1_finite_differences_of_the_ot_value():
    X, Y, a, b = _problem(11, 6, 5, 2)
    eps = 0.6
    f, g = _converged(X, Y, a, b, eps)
    gX, gY = oracle.gradient(X, Y, a, b, f, g, eps)
    h = 1e-5
    for i, k in itertools.product(range(X.shape[0]), range(X.shape[1])):
        Xp, Xm = X.copy(), X.copy()
        Xp[i, k] += h
        Xm[i, k] -= h
        fd = (_ot_value(Xp, Y, a, b, eps) - _ot_value(Xm, Y, a, b, eps)) / (2 * h)
        assert abs(fd - gX[i, k]) <= 1e-6 * (1 + abs(gX[i, k])), (i, k, fd, gX[i, k])
    for j, k in itertools.product(range(Y.shape[0]), range(Y.shape[1])):
        Yp, Ym = Y.copy(), Y.copy()
        Yp[j, k] += h
        Ym[j, k] -= h
        fd = (_ot_value(X, Yp, a, b, eps) - _ot_value(X, Ym, a, b, eps)) / (2 * h)
        assert abs(fd - gY[j, k]) <= 1e-6 * (1 + abs(gY[j, k])), (j, k, fd, gY[j, k])


def test_g2_finite_differences_of_the_dual_at_fixed_potentials():
    X, Y, a, b = _problem(12, 7, 4, 3)
    eps = 0.4
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=2)  # far from converged
    f, g = r["f"], r["g"]
    gX, gY = oracle.gradient(X, Y, a, b, f, g, eps)
    h = 1e-6
    for i, k in [(0, 0), (3, 2), (6, 1)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[i, k] += h
        Xm[i, k] -= h
        fd = (oracle.dual_objective(Xp, Y, a, b, f, g, eps) -
              oracle.dual_objective(Xm, Y, a, b, f, g, eps)) / (2 * h)
        assert abs(fd - gX[i, k]) <= 1e-7 * (1 + abs(gX[i, k]))
    for j, k in [(0, 1), (3, 0)]:
        Yp, Ym = Y.copy(), Y.copy()
        Yp[j, k] += h
        Ym[j, k] -= h
        fd = (oracle.dual_objective(X, Yp, a, b, f, g, eps) -
              oracle.dual_objective(X, Ym, a, b, f, g, eps)) / (2 * h)
        assert abs(fd - gY[j, k]) <= 1e-7 * (1 + abs(gY[j, k]))


def test_g3_translation_invariance():
    X, Y, a, b = _problem(13, 9, 11, 4)
    rng = np.random.default_rng(5)
    f = rng.standard_normal(9)
    g = rng.standard_normal(11)
    gX, gY = oracle.gradient(X, Y, a, b, f, g, 0.7)
    scale = np.abs(gX).sum() + np.abs(gY).sum()
    assert np.max(np.abs(gX.sum(0) + gY.sum(0))) <= 1e-13 * scale


def test_g4_single_target_closed_form():
    X, Y, a, b = _problem(14, 8, 1, 3)
    eps = 0.3
    f, g = _converged(X, Y, a, b, eps)
    gX, gY = oracle.gradient(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(gX, 2 * a[:, None] * (X - Y[0]), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gY[0], 2 * (a[:, None] * (Y[0] - X)).sum(0), rtol=1e-11,
                               atol=1e-13)


def test_g5_dual_objective_after_updates_and_assignment_brackets():
    X, Y, a, b = _problem(15, 6, 8, 2)
    r = oracle.sinkhorn(X, Y, a, b, eps=0.5, iters=3)
    D = oracle.dual_objective(X, Y, a, b, r["f"], r["g"], 0.5)
    assert abs(D - (a @ r["f"] + b @ r["g"])) <= 1e-13 * (1 + abs(D))
    # uniform n = m = 5: W <= OT_eps <= W + eps log n (brute force over 5! plans)
    rng = np.random.default_rng(16)
    n = 5
    Xs = rng.standard_normal((n, 2))
    Ys = rng.standard_normal((n, 2)) + 0.5
    u = np.full(n, 1.0 / n)
    C = ((Xs[:, None, :] - Ys[None, :, :]) ** 2).sum(-1)
    W = min(C[np.arange(n), list(p)].mean() for p in itertools.permutations(range(n)))
    eps = 0.25
    f, g = _converged(Xs, Ys, u, u, eps)
    D = oracle.dual_objective(Xs, Ys, u, u, f, g, eps)
    assert W - 1e-12 <= D <= W + eps * np.log(n) + 1e-12


def test_g6_column_transport_is_the_transposed_plan():
    X, Y, a, b = _problem(17, 7, 9, 3)
    eps = 0.5
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=5)
    f, g = r["f"], r["g"]
    C = ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)
    P = a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)
    W = np.random.default_rng(3).standard_normal((7, 4))
    np.testing.assert_allclose(oracle.transport_t(X, Y, a, b, f, g, W, eps), P.T @ W,
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.transport_t(X, Y, a, b, f, g, W, eps, divide_by_b=True),
                               (P.T @ W) / b[:, None], rtol=1e-12, atol=1e-14)
    cols = [0, 4, 8]
    np.testing.assert_allclose(oracle.transport_t(X, Y, a, b, f, g, W, eps, cols=cols),
                               (P.T @ W)[cols], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mutant", ["no_factor_2", "sign"])
def test_pins_catch_planted_gradient_mistakes(mutant):
    # A plausible slip, planted in a copy of the oracle's result on the CPU:
    # G4's closed form (and G3's sum) reject it.
    X, Y, a, b = _problem(14, 8, 1, 3)
    f, g = _converged(X, Y, a, b, 0.3)
    gX, _ = oracle.gradient(X, Y, a, b, f, g, 0.3)
    bad = gX / 2 if mutant == "no_factor_2" else -gX
    with pytest.raises(AssertionError):
        np.testing.assert_allclose(bad, 2 * a[:, None] * (X - Y[0]), rtol=1e-11, atol=1e-13)


def _normalise(P):
    return P / np.linalg.norm(P, axis=1, keepdims=True)


def _cosine_gradient(X, Y, a, b, f, g, eps):
    """The gradient for C = 2 - 2 cos, from the oracle's gradient with respect
    to the normalised points taken back through x -> x/|x| (Jacobian
    (I - x^ x^T)/|x|)."""
    Xn, Yn = _normalise(X), _normalise(Y)
    gXn, gYn = oracle.gradient(Xn, Yn, a, b, f, g, eps)

    def back(P, Pn, G):
        return (G - Pn * np.sum(Pn * G, axis=1, keepdims=True)) / np.linalg.norm(
            P, axis=1, keepdims=True)

    return back(X, Xn, gXn), back(Y, Yn, gYn)


def test_g7_cosine_cost_chain_rule_by_finite_differences():
    # OT with C = 2 - 2 cos(x, y) is the squared-Euclidean OT of the
    # normalised clouds; its gradient with respect to the raw points, by
    # central differences of the converged value, matches the chain rule.
    X, Y, a, b = _problem(18, 5, 6, 3)
    eps = 0.3
    f, g = _converged(_normalise(X), _normalise(Y), a, b, eps)
    C = 2.0 - 2.0 * (_normalise(X) @ _normalise(Y).T)
    np.testing.assert_allclose(C, ((_normalise(X)[:, None] - _normalise(Y)[None]) ** 2).sum(-1),
                               atol=1e-14)
    gX, gY = _cosine_gradient(X, Y, a, b, f, g, eps)
    h = 1e-5

    def val(Xq, Yq):
        return _ot_value(_normalise(Xq), _normalise(Yq), a, b, eps)

    for i, k in [(0, 0), (2, 1), (4, 2)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[i, k] += h
        Xm[i, k] -= h
        fd = (val(Xp, Y) - val(Xm, Y)) / (2 * h)
        assert abs(fd - gX[i, k]) <= 1e-6 * (1 + abs(gX[i, k]))
    for j, k in [(1, 0), (5, 2)]:
        Yp, Ym = Y.copy(), Y.copy()
        Yp[j, k] += h
        Ym[j, k] -= h
        fd = (val(X, Yp) - val(X, Ym)) / (2 * h)
        assert abs(fd - gY[j, k]) <= 1e-6 * (1 + abs(gY[j, k]))
    # scale invariance of the cosine cost: the gradient is orthogonal to x_i
    assert np.max(np.abs(np.sum(gX * X, axis=1))) <= 1e-12
