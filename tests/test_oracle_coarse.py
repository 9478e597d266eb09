"""Pins of the coarse-stage oracle (oracle/coarse.py).

C1  centroids conserve the weight and the first moment of every cell, and a
    cell of copies of one point has that point as centroid;
C2  one-point cells reproduce the fine problem: the lift of the coarse
    potentials equals the fine solve's potentials;
C3  the sampled check over every row and column equals the full L1 marginal
    residual of the lifted potentials, each side divided by its total mass;
C4  the coarse start on a Morton-ordered pair passes a loose check, and a
    strict one uses up its rounds (the loop runs and reports rejection);
C5  a planted slip (the unweighted mean as centroid) breaks C1.
"""
import numpy as np
import pytest

import oracle
from oracle import blocksparse as obs
from oracle import coarse as oc


def _pair(seed, n, m, d=3):
    rng = np.random.default_rng(seed)
    X = rng.uniform(0, 1, (n, d))
    Y = rng.uniform(0, 1, (m, d)) * 0.9 + 0.05
    X, Y = X[obs.morton_order(X)], Y[obs.morton_order(Y)]
    a, b = rng.standard_exponential(n), rng.standard_exponential(m)
    return X, Y, a / a.sum(), b / b.sum()


def test_c1_centroid_sums():
    X, Y, a, b = _pair(1, 301, 250)
    C, W = oc.centroids(X, a, 16)
    assert len(C) == (301 + 15) // 16
    for k in range(len(C)):
        sl = slice(16 * k, 16 * k + 16)
        assert W[k] == pytest.approx(a[sl].sum(), rel=1e-14)
        np.testing.assert_allclose(W[k] * C[k], (a[sl, None] * X[sl]).sum(0), rtol=1e-13)
    P = np.repeat(X[:3], 5, axis=0)
    C, W = oc.centroids(P, np.arange(1, 16, dtype=float), 5)
    np.testing.assert_allclose(C, X[:3], rtol=1e-14)


def test_c2_one_point_cells_are_the_fine_problem():
    X, Y, a, b = _pair(2, 120, 100)
    res = oc.coarse_start(X, Y, a, b, 1, 0.05, 60, tol=1e9, max_rounds=1)
    ref = oracle.sinkhorn(X, Y, a, b, eps=0.05, iters=60)
    np.testing.assert_allclose(res["f"], ref["f"], atol=1e-12)
    np.testing.assert_allclose(res["g"], ref["g"], atol=1e-12)


def test_c3_full_sample_is_the_marginal_residual():
    X, Y, a, b = _pair(3, 200, 170)
    eps = 0.03
    res = oc.coarse_start(X, Y, a, b, 8, eps, 40, tol=1e9, max_rounds=1)
    er, ec = oc.sampled_marginal_error(X, Y, a, b, res["f"], res["g"], eps, np.arange(200),
                                       np.arange(170))
    full = oracle.marginal_residual(X, Y, a, b, res["f"], res["g"], eps)
    assert er == pytest.approx(full[1], rel=1e-9)  # total mass 1 on each side
    assert ec == pytest.approx(full[2], rel=1e-9)


def test_c4_rounds_run_and_pass():
    X, Y, a, b = _pair(4, 800, 700)
    rng = np.random.default_rng(5)
    rows, cols = rng.choice(800, 64, replace=False), rng.choice(700, 64, replace=False)
    # (the lift copies a cell's potential to its points, so its error is set by
    # the cell size against sqrt(eps), which more coarse iterations do not
    # reduce: a loose tolerance passes, a strict one runs out of rounds)
    res = oc.coarse_start(X, Y, a, b, 4, 0.05, 30, n_stages=4, eps_start=0.2, more_iters=20,
                          tol=0.3, max_rounds=4, rows=rows, cols=cols)
    assert res["accepted"] and 1 <= res["rounds"] <= 4
    strict = oc.coarse_start(X, Y, a, b, 4, 0.05, 30, n_stages=4, eps_start=0.2, more_iters=20,
                             tol=1e-9, max_rounds=3, rows=rows, cols=cols)
    assert not strict["accepted"] and strict["rounds"] == 3


def test_c5_unweighted_mean_slip_is_caught(monkeypatch):
    X, Y, a, b = _pair(6, 64, 40)

    def unweighted(P, w, cell):
        nc = (len(P) + cell - 1) // cell
        return (np.stack([P[k * cell:(k + 1) * cell].mean(0) for k in range(nc)]),
                np.array([w[k * cell:(k + 1) * cell].sum() for k in range(nc)]))

    C, W = unweighted(X, a, 16)
    bad = max(np.abs(W[k] * C[k] - (a[16 * k:16 * k + 16, None] * X[16 * k:16 * k + 16]).sum(0)).max()
              for k in range(len(C)))
    assert bad > 1e-6
