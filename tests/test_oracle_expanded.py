"""Pins of oracle/expanded.py (the matrix-product form of the float64 oracle
used for the full-size stored values of the 50k recipes) to the
direct-difference oracle, which is itself pinned to the mathematics in
test_oracle_pins.py.

Every recipe's distribution, schedule and weights at a reduced size: the two
forms agree iterate for iterate within 1e-11 eps (float64 rounding of the
expansion, about 1e-16 (|x|^2 + |y|^2) per cost entry).  A planted slip in
each ingredient of the expansion (the factor 2 of the cross term, a squared
norm, the weight term) is caught by the same comparison.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import expanded
from streaming_sinkhorn_solver_amd import workloads

CASES = [("c1", dict(n=300, m=257), 30), ("c2", dict(n=500, m=400), 20),
         ("c3", dict(n=400, m=350, d=96), 15), ("c4", dict(n=300, m=250, d=200), 3),
         ("c5", dict(n=700, m=650), 10)]


@pytest.mark.parametrize("name,kw,iters", CASES)
def test_expanded_matches_direct_differences(name, kw, iters):
    w = workloads.make(name, **kw)
    r1 = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=iters, n_stages=w.n_stages,
                         eps_start=w.eps_start)
    seen = []
    r2 = expanded.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=iters, n_stages=w.n_stages,
                           eps_start=w.eps_start,
                           on_iteration=lambda k, e, f, g: seen.append((k, e)))
    assert r2["iters"] == iters * w.n_stages == len(seen)
    assert seen[-1][1] == pytest.approx(w.eps, rel=1e-12)
    assert np.max(np.abs(r1["f"] - r2["f"])) <= 1e-11 * w.eps
    assert np.max(np.abs(r1["g"] - r2["g"])) <= 1e-11 * w.eps


def test_single_updates_match():
    w = workloads.make("c3", n=300, m=280, d=64)
    g = np.random.default_rng(5).normal(0, 0.05, w.m)
    f = np.random.default_rng(6).normal(0, 0.05, w.n)
    assert np.max(np.abs(expanded.f_update(w.X, w.Y, w.b, g, w.eps) -
                         oracle.f_update(w.X, w.Y, w.b, g, w.eps))) <= 1e-12 * w.eps
    assert np.max(np.abs(expanded.g_update(w.X, w.Y, w.a, f, w.eps) -
                         oracle.g_update(w.X, w.Y, w.a, f, w.eps))) <= 1e-12 * w.eps


@pytest.mark.parametrize("slip", ["cross_factor", "row_norm", "weight"])
def test_planted_slips_are_caught(monkeypatch, slip):
    """A copy of the soft-min with one ingredient wrong disagrees with the
    direct-difference oracle far beyond the 1e-11 eps pin."""

    def bad_soft_min(P, pn, Q, qn, logw, pot, eps):
        cross = 1.0 if slip == "cross_factor" else 2.0
        pn_ = 0.0 * pn if slip == "row_norm" else pn
        lw = 0.0 * logw if slip == "weight" else logw
        C = pn_[:, None] + qn[None, :] - cross * (P @ Q.T)
        z = (pot[None, :] - C) / eps + lw[None, :]
        return -eps * torch.logsumexp(z, dim=1)

    monkeypatch.setattr(expanded, "_soft_min", bad_soft_min)
    w = workloads.make("c3", n=200, m=180, d=32)
    r1 = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=3)
    r2 = expanded.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=3)
    assert np.max(np.abs(r1["f"] - r2["f"])) > 1e-3 * w.eps
