"""The stored oracle snapshots still match the live oracle bit for bit."""
import os

import numpy as np

import oracle
from streaming_sinkhorn_solver_amd import workloads

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    return np.loadtxt(os.path.join(HERE, name))


def test_c1_snapshots_match_live_oracle():
    w = workloads.make("c1")
    for iters in (1, 100):
        res = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=iters)
        np.testing.assert_array_equal(res["f"], load(f"c1_oracle_f_iter{iters}.txt"))
        np.testing.assert_array_equal(res["g"], load(f"c1_oracle_g_iter{iters}.txt"))
    tot, rt, ct = load("c1_oracle_residual_iter100.txt")
    res = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=100)
    live = oracle.marginal_residual(w.X, w.Y, w.a, w.b, res["f"], res["g"], w.eps)
    np.testing.assert_allclose(live, (tot, rt, ct), rtol=1e-12, atol=1e-18)


def test_generator_is_deterministic():
    a1 = workloads.make("c3", n=300, m=200)
    a2 = workloads.make("c3", n=300, m=200)
    for k in ("X", "Y", "a", "b"):
        np.testing.assert_array_equal(getattr(a1, k), getattr(a2, k))
        assert getattr(a1, k).dtype == np.float32
    assert abs(float(a1.a.astype(np.float64).sum()) - 1.0) < 1e-5
    w4 = workloads.make("c4", n=64, m=48, d=128)
    np.testing.assert_allclose(np.linalg.norm(w4.X.astype(np.float64), axis=1), 1.0, rtol=1e-6)
    assert w4.V.shape == (48, 128) and w4.n_stages == 10 and w4.eps_start == 1.0
