"""Pins of the float64 CPU oracle against facts fixed by the mathematics.

The pages (FlashSinkhorn explainer, "Method" part 1) define the update
    f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j],   C_ij = |x_i - y_j|^2,
and its mirror for g; they print no worked example, potential or plan.  So
the oracle is pinned here by things it does not compute itself:

P1  dense scaling-form Sinkhorn (u = a/Kv, v = b/K^T u) iterate for iterate;
P2  brute-force optimal assignment (and scipy's assignment solver): duality
    brackets W <= OT_eps <= W + eps log n, and P -> sigma*/n as eps -> 0;
P3  1-D sorted matching at n = 1024;
P4  soft-min brackets (min / Jensen / Hoeffding) after every f-update;
P5  closed forms (a single target point; coincident clouds; 2-point case);
P6  exact marginals after each half-step;
P7  monotone dual ascent;
P8  symmetric problem: f - g constant, (f+g)/2 the averaged fixed point;
P9  translation covariance of every iterate;
P10 power-of-two scaling (2X, 2Y, 4 eps) -> (4f, 4g), bit for bit;
P11 row permutation; P12 duplicate split; P13 large-eps limit;
plus the transport product and the residual against a dense plan, and the
annealing schedule's end points.

Each one would catch a plausible slip in the oracle (a dropped log-weight, a
sign, a swapped a/b, a transposed cost, a missing 1/eps).
"""
import itertools

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment

import oracle
from streaming_sinkhorn_solver_amd import workloads


def dense_cost(X, Y):
    X = np.asarray(X, np.float64)
    Y = np.asarray(Y, np.float64)
    diff = X[:, None, :] - Y[None, :, :]
    return np.einsum("ijk,ijk->ij", diff, diff)


def dense_plan(X, Y, a, b, f, g, eps):
    C = dense_cost(X, Y)
    return np.asarray(a)[:, None] * np.asarray(b)[None, :] * np.exp(
        (np.asarray(f)[:, None] + np.asarray(g)[None, :] - C) / eps)


def exp_weights(rng, k):
    e = rng.standard_exponential(k)
    return e / e.sum()


def small_problem(seed, n, m, d, weights="exp", offset=0.3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d)) * 0.8 + offset
    if weights == "exp":
        a, b = exp_weights(rng, n), exp_weights(rng, m)
    else:
        a, b = np.full(n, 1.0 / n), np.full(m, 1.0 / m)
    return X, Y, a, b


# --------------------------------------------------------------------- P1
@pytest.mark.parametrize("seed,n,m,d,eps_rel", [(0, 17, 23, 3, 0.3), (1, 40, 31, 5, 0.1),
                                                (2, 64, 64, 2, 0.05), (3, 9, 50, 8, 1.0)])
def test_p1_scaling_form_iterate_for_iterate(seed, n, m, d, eps_rel):
    X, Y, a, b = small_problem(seed, n, m, d)
    C = dense_cost(X, Y)
    eps = eps_rel * np.median(C)
    K = np.exp(-C / eps)
    v = b.copy()  # g = 0
    g = np.zeros(m)
    for _ in range(12):
        u = a / (K @ v)
        f_ref = eps * np.log(u / a)
        f = oracle.f_update(X, Y, b, g, eps)
        np.testing.assert_allclose(f, f_ref, rtol=1e-10, atol=1e-10 * np.abs(f_ref).max())
        v = b / (K.T @ u)
        g_ref = eps * np.log(v / b)
        g = oracle.g_update(X, Y, a, f, eps)
        np.testing.assert_allclose(g, g_ref, rtol=1e-10, atol=1e-10 * np.abs(g_ref).max())
    # the driver runs exactly these steps
    res = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=12)
    np.testing.assert_array_equal(res["f"], f)
    np.testing.assert_array_equal(res["g"], g)


# --------------------------------------------------------------------- P2
def brute_force_assignment(C):
    n = C.shape[0]
    best, arg = np.inf, None
    for perm in itertools.permutations(range(n)):
        v = C[np.arange(n), perm].mean()
        if v < best:
            best, arg = v, perm
    return best, np.array(arg)


@pytest.mark.parametrize("seed,n", [(11, 5), (13, 7), (14, 7), (15, 6)])
def test_p2_brute_force_assignment_brackets(seed, n):
    X, Y, a, b = small_problem(seed, n, n, 2, weights="uniform")
    C = dense_cost(X, Y)
    W, perm = brute_force_assignment(C)
    r, c = linear_sum_assignment(C)
    assert abs(C[r, c].mean() - W) < 1e-12
    for eps_rel in (0.5, 0.1):
        eps = eps_rel * np.median(C)
        res = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=50000, tol=1e-10, check_every=50)
        f, g = res["f"], res["g"]
        tot, _, _ = oracle.marginal_residual(X, Y, a, b, f, g, eps)
        assert tot <= 1e-10
        dual = a @ f + b @ g
        P = dense_plan(X, Y, a, b, f, g, eps)
        primal_cost = (P * C).sum()
        slack = 1e-9
        assert W - slack <= dual <= W + eps * np.log(n) + slack
        assert W - slack <= primal_cost <= W + eps * np.log(n) + slack
    # eps -> 0 (annealed from median C to 1e-3 median C): the plan
    # concentrates on the optimal permutation
    eps_end = 1e-3 * np.median(C)
    res = oracle.sinkhorn(X, Y, a, b, eps=eps_end, eps_start=np.median(C), n_stages=30,
                          iters=400)
    P = dense_plan(X, Y, a, b, res["f"], res["g"], eps_end)
    target = np.zeros((n, n))
    target[np.arange(n), perm] = 1.0 / n
    assert np.abs(P - target).max() < 1e-6


def test_p2_assignment_solver_bracket_n200():
    X, Y, a, b = small_problem(13, 200, 200, 3, weights="uniform")
    C = dense_cost(X, Y)
    r, c = linear_sum_assignment(C)
    W = C[r, c].mean()
    eps = 0.05 * np.median(C)
    res = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=5000, tol=1e-9, check_every=25)
    assert res["residual"] <= 1e-9
    dual = a @ res["f"] + b @ res["g"]
    assert W - 1e-9 <= dual <= W + eps * np.log(200) + 1e-9


# --------------------------------------------------------------------- P3
def test_p3_one_dimensional_sorted_matching():
    rng = np.random.default_rng(20)
    n = 1024
    X = rng.standard_normal((n, 1))
    Y = rng.standard_normal((n, 1)) * 1.5 + 0.7
    a = np.full(n, 1.0 / n)
    W = np.mean((np.sort(X[:, 0]) - np.sort(Y[:, 0])) ** 2)
    eps = 0.02
    res = oracle.sinkhorn(X, Y, a, a, eps=eps, iters=4000, tol=1e-7, check_every=20)
    assert 0 < res["residual"] <= 1e-7
    dual = a @ res["f"] + a @ res["g"]
    assert W - 1e-7 <= dual <= W + eps * np.log(n) + 1e-7


# --------------------------------------------------------------------- P4
@pytest.mark.parametrize("seed", [30, 31])
def test_p4_softmin_brackets_every_f_update(seed):
    X, Y, a, b = small_problem(seed, 37, 45, 4)
    C = dense_cost(X, Y)
    rng = np.random.default_rng(seed)
    for eps in (0.01, 0.3, 5.0):
        for _ in range(3):
            g = rng.standard_normal(45) * 2.0
            f = oracle.f_update(X, Y, b, g, eps)
            h = C - g[None, :]
            tol = 1e-12 * (1 + np.abs(h).max())
            assert np.all(f >= h.min(1) - tol)
            assert np.all(f <= (h - eps * np.log(b)[None, :]).min(1) + tol)
            mean_h = h @ b
            R = h.max(1) - h.min(1)
            assert np.all(f <= mean_h + tol)
            assert np.all(f >= mean_h - R ** 2 / (8 * eps) - tol)


# --------------------------------------------------------------------- P5
def test_p5_single_target_point():
    rng = np.random.default_rng(40)
    X = rng.standard_normal((11, 3))
    Y = rng.standard_normal((1, 3))
    a = exp_weights(rng, 11)
    b = np.array([1.0])
    res = oracle.sinkhorn(X, Y, a, b, eps=0.07, iters=3)
    np.testing.assert_allclose(res["f"], dense_cost(X, Y)[:, 0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(res["g"], [0.0], atol=1e-13)


def test_p5_coincident_clouds():
    x0 = np.array([0.3, -1.2, 2.0])
    y0 = np.array([1.1, 0.4, -0.5])
    X = np.tile(x0, (6, 1))
    Y = np.tile(y0, (9, 1))
    rng = np.random.default_rng(41)
    a, b = exp_weights(rng, 6), exp_weights(rng, 9)
    res = oracle.sinkhorn(X, Y, a, b, eps=0.2, iters=4)
    c = np.sum((x0 - y0) ** 2)
    np.testing.assert_allclose(res["f"], c, rtol=1e-13)
    np.testing.assert_allclose(res["g"], 0.0, atol=1e-12)


def test_p5_two_point_closed_form():
    # x = {0, 1}, y = {0, 1} on a line, uniform weights: C = [[0,1],[1,0]].
    X = np.array([[0.0], [1.0]])
    Y = X.copy()
    a = np.array([0.5, 0.5])
    eps = 0.25
    res = oracle.sinkhorn(X, Y, a, a, eps=eps, iters=1)
    f_exp = -eps * np.log(0.5 * (1.0 + np.exp(-1.0 / eps)))
    np.testing.assert_allclose(res["f"], [f_exp, f_exp], rtol=1e-14)
    np.testing.assert_allclose(res["g"], [0.0, 0.0], atol=1e-14)
    # the plan puts p = 1/(2(1+e^{-1/eps})) on the diagonal
    P = dense_plan(X, Y, a, a, res["f"], res["g"], eps)
    np.testing.assert_allclose(np.diag(P), 0.5 / (1 + np.exp(-1 / eps)), rtol=1e-13)


# --------------------------------------------------------------- P6 and P7
@pytest.mark.parametrize("seed", [50, 51])
def test_p6_p7_marginals_and_dual_ascent(seed):
    X, Y, a, b = small_problem(seed, 30, 26, 3)
    C = dense_cost(X, Y)
    eps = 0.2 * np.median(C)
    f, g = np.zeros(30), np.zeros(26)
    last = -np.inf

    def dual(f, g):
        P = dense_plan(X, Y, a, b, f, g, eps)
        return a @ f + b @ g - eps * (P.sum() - a.sum() * b.sum())

    for _ in range(15):
        f = oracle.f_update(X, Y, b, g, eps)
        P = dense_plan(X, Y, a, b, f, g, eps)
        np.testing.assert_allclose(P.sum(1), a, rtol=1e-12)
        D = dual(f, g)
        assert D >= last - 1e-13
        last = D
        g = oracle.g_update(X, Y, a, f, eps)
        P = dense_plan(X, Y, a, b, f, g, eps)
        np.testing.assert_allclose(P.sum(0), b, rtol=1e-12)
        D = dual(f, g)
        assert D >= last - 1e-13
        last = D
    # the driver's dual log is <a,f> + <b,g> after each half-step
    res = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=15, log_dual=True)
    assert np.all(np.diff(res["dual"]) >= -1e-13)


# --------------------------------------------------------------------- P8
def test_p8_symmetric_problem():
    rng = np.random.default_rng(60)
    X = rng.standard_normal((25, 3))
    a = exp_weights(rng, 25)
    C = dense_cost(X, X)
    eps = 0.3 * np.median(C)
    res = oracle.sinkhorn(X, X, a, a, eps=eps, iters=3000, tol=1e-13, check_every=10)
    f, g = res["f"], res["g"]
    diff = f - g
    assert np.ptp(diff) < 1e-9
    # averaged fixed point h = (h + T(h))/2, T(h)_i = -eps log sum_j a_j e^{(h_j - C_ij)/eps}
    h = np.zeros(25)
    for _ in range(5000):
        Th = -eps * np.log(np.exp((h[None, :] - C) / eps) @ a)
        h = 0.5 * (h + Th)
    np.testing.assert_allclose(0.5 * (f + g), h, atol=1e-9)


# --------------------------------------------------------------------- P9
def test_p9_translation_every_iterate():
    X, Y, a, b = small_problem(70, 21, 34, 3)
    t = np.array([0.7, -1.3, 0.25])
    eps = 0.15
    Yt = Y + t
    for iters in (1, 2, 7):
        ref = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=iters)
        g0 = 2 * Y @ t + t @ t
        sh = oracle.sinkhorn(X, Yt, a, b, eps=eps, iters=iters, g0=g0)
        np.testing.assert_allclose(sh["f"], ref["f"] - 2 * X @ t, atol=1e-10)
        np.testing.assert_allclose(sh["g"], ref["g"] + 2 * Y @ t + t @ t, atol=1e-10)


# -------------------------------------------------------------------- P10
def test_p10_power_of_two_scaling_bit_exact():
    X, Y, a, b = small_problem(80, 19, 27, 3)
    eps = 0.11
    ref = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=9)
    sc = oracle.sinkhorn(2 * X, 2 * Y, a, b, eps=4 * eps, iters=9)
    np.testing.assert_array_equal(sc["f"], 4 * ref["f"])
    np.testing.assert_array_equal(sc["g"], 4 * ref["g"])


# -------------------------------------------------------------------- P11
def test_p11_row_permutation():
    X, Y, a, b = small_problem(90, 33, 28, 4)
    perm = np.random.default_rng(91).permutation(33)
    eps = 0.2
    ref = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=6)
    pr = oracle.sinkhorn(X[perm], Y, a[perm], b, eps=eps, iters=6)
    np.testing.assert_allclose(pr["f"], ref["f"][perm], atol=1e-12)
    np.testing.assert_allclose(pr["g"], ref["g"], atol=1e-12)
    # first f-update depends on the row only: bit-identical
    f1 = oracle.f_update(X, Y, b, np.zeros(28), eps)
    f1p = oracle.f_update(X[perm], Y, b, np.zeros(28), eps)
    np.testing.assert_array_equal(f1p, f1[perm])


# -------------------------------------------------------------------- P12
def test_p12_duplicate_split():
    X, Y, a, b = small_problem(100, 15, 12, 3)
    j = 5
    Y2 = np.vstack([Y, Y[j:j + 1]])
    b2 = np.concatenate([b, [b[j] / 2]])
    b2[j] = b[j] / 2
    eps = 0.3
    ref = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=8)
    dup = oracle.sinkhorn(X, Y2, a, b2, eps=eps, iters=8)
    np.testing.assert_allclose(dup["f"], ref["f"], atol=1e-12)
    np.testing.assert_allclose(dup["g"][:12], ref["g"], atol=1e-12)
    np.testing.assert_allclose(dup["g"][12], ref["g"][j], atol=1e-12)


# -------------------------------------------------------------------- P13
def test_p13_large_eps_limit():
    X, Y, a, b = small_problem(110, 14, 16, 3)
    C = dense_cost(X, Y)
    for eps in (1e4, 1e6):
        f = oracle.f_update(X, Y, b, np.zeros(16), eps)
        np.testing.assert_allclose(f, C @ b, atol=10 * C.max() ** 2 / eps)


# ------------------------------------------------------ residual, transport
def test_residual_and_transport_against_dense_plan():
    X, Y, a, b = small_problem(120, 23, 19, 3)
    rng = np.random.default_rng(121)
    f = rng.standard_normal(23) * 0.1
    g = rng.standard_normal(19) * 0.1
    V = rng.standard_normal((19, 5))
    eps = 0.4
    P = dense_plan(X, Y, a, b, f, g, eps)
    tot, rt, ct = oracle.marginal_residual(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(rt, np.abs(P.sum(1) - a).sum(), rtol=1e-12)
    np.testing.assert_allclose(ct, np.abs(P.sum(0) - b).sum(), rtol=1e-12)
    np.testing.assert_allclose(tot, rt + ct, rtol=1e-15)
    U = oracle.transport(X, Y, a, b, f, g, V, eps)
    np.testing.assert_allclose(U, P @ V, rtol=1e-12, atol=1e-15)
    T = oracle.transport(X, Y, a, b, f, g, V, eps, divide_by_a=True)
    np.testing.assert_allclose(T, (P @ V) / a[:, None], rtol=1e-12, atol=1e-15)
    rows = [3, 0, 22]
    Ur = oracle.transport(X, Y, a, b, f, g, V, eps, rows=rows)
    np.testing.assert_array_equal(Ur, U[rows])


def test_subset_updates_match_full():
    X, Y, a, b = small_problem(130, 40, 35, 6)
    rng = np.random.default_rng(131)
    g = rng.standard_normal(35)
    f = rng.standard_normal(40)
    rows = [39, 0, 17, 17]
    cols = [0, 34, 2]
    np.testing.assert_array_equal(oracle.f_update_rows(X, Y, b, g, 0.3, rows),
                                  oracle.f_update(X, Y, b, g, 0.3)[rows])
    np.testing.assert_array_equal(oracle.g_update_cols(X, Y, a, f, 0.3, cols),
                                  oracle.g_update(X, Y, a, f, 0.3)[cols])


def test_annealing_schedule_end_points():
    assert oracle.stage_eps(0, 10, 1.0, 0.01) == 1.0
    assert abs(oracle.stage_eps(9, 10, 1.0, 0.01) - 0.01) < 1e-15
    assert abs(oracle.stage_eps(3, 10, 1.0, 0.01) - 10 ** (-6 / 9)) < 1e-15
    assert oracle.stage_eps(0, 1, 5.0, 0.2) == 0.2
    # a one-stage run at eps equals the annealed run's last stage when it has one stage
    X, Y, a, b = small_problem(140, 12, 10, 2)
    r1 = oracle.sinkhorn(X, Y, a, b, eps=0.3, iters=5)
    r2 = oracle.sinkhorn(X, Y, a, b, eps=0.3, eps_start=9.0, n_stages=1, iters=5)
    np.testing.assert_array_equal(r1["f"], r2["f"])


def test_tol_stop_returns_measured_state():
    X, Y, a, b = small_problem(150, 30, 30, 3)
    res = oracle.sinkhorn(X, Y, a, b, eps=0.5, iters=1000, tol=1e-8, check_every=5)
    assert res["iters"] % 5 == 0 and res["iters"] < 1000
    tot, _, _ = oracle.marginal_residual(X, Y, a, b, res["f"], res["g"], 0.5)
    assert tot == pytest.approx(res["residual"], rel=1e-12)
    assert tot <= 1e-8


def test_small_configs_converge_below_1e6():
    # The small recipes, driven to the 1e-6 marginal residual.
    for name, size in (("c1", 256), ("c2", 300), ("c3", 300), ("c5", 400)):
        w = workloads.make(name, n=size, m=size - 17)
        res = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=max(w.eps, 0.05), iters=20000,
                              tol=1e-6, check_every=20)
        assert 0 <= res["residual"] <= 1e-6, (name, res["residual"])
