"""The single-launch solve of small d <= 8 problems (fs_persistent.hip): the
whole schedule in one launch, both clouds in each workgroup's LDS, a grid
barrier between half-steps, fp32 vector scores.  Against the float64 oracle
after the same iterations at the fp32 bar (1e-3 eps), on every d from 1 to 8,
ragged sizes (rows per workgroup from 1 to 16, lane groups from 64 to 4,
workgroups with no rows, unequal clouds), annealed schedules, a warm start,
and at each d's size limit (n + m: 2389 for d <= 3, 1433 for d <= 7, 1024 for
d = 8); against the multi-launch path on the same problem (same bar); and one
point past each limit, where the multi-launch path runs."""
import numpy as np
import pytest

from helpers import dev, host, max_err, oracle_solve
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _solve(w, eps, iters, single, n_stages=1, eps_start=None, g0=None):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    f = torch.zeros(w.n, device="cuda")
    g = torch.zeros(w.m, device="cuda") if g0 is None else dev(g0)
    p = binding.fs_potentials_init(dev(w.X), dev(w.Y), dev(w.a), dev(w.b), f=f,
                                   g=None if g0 is not None else g)
    if g0 is not None:
        g.copy_(dev(g0))
    info = binding.fs_sinkhorn_solve(p, f, g, eps_end=eps, eps_start=eps_start,
                                     n_stages=n_stages, iters_per_stage=iters,
                                     warm_start=g0 is not None, single_launch=single,
                                     time_kernels=True)
    torch.cuda.synchronize()
    return host(f), host(g), info


@pytest.mark.parametrize("d", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,m", [(300, 257), (600, 411), (40, 960), (1, 5)])
def test_single_launch_against_oracle(fs, d, n, m):
    w = workloads.random_cloud(600 + d + n, n, m, d, weights="exp", scale=1.0 / np.sqrt(d))
    eps = 0.2
    f, g, info = _solve(w, eps, 12, 1)
    assert info["single_launch"]
    assert info["lse_launches"] == 24  # one launch, reported as its half-steps
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=eps, iters=12)
    assert max_err(f, ref["f"]) <= TOL * eps and max_err(g, ref["g"]) <= TOL * eps
    f2, g2, info2 = _solve(w, eps, 12, -1)
    assert not info2["single_launch"]
    assert max_err(f, f2) <= TOL * eps and max_err(g, g2) <= TOL * eps


def test_c1_recipe_single_launch(fs):
    # the 512 x 512, 3-D recipe takes the single launch by default; without a
    # warm start it starts from g = 0 whatever f and g held before
    import torch

    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make("c1")
    f = torch.full((w.n,), float("nan"), device="cuda")
    g = torch.full((w.m,), float("nan"), device="cuda")
    p = binding.fs_potentials_init(dev(w.X), dev(w.Y), dev(w.a), dev(w.b))
    info = binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=w.iters)
    torch.cuda.synchronize()
    assert info["single_launch"]
    f, g = host(f), host(g)
    import os

    gold = os.path.join(os.path.dirname(__file__), "golden")
    assert max_err(f, np.loadtxt(os.path.join(gold, "c1_oracle_f_iter100.txt"))) <= TOL * w.eps
    assert max_err(g, np.loadtxt(os.path.join(gold, "c1_oracle_g_iter100.txt"))) <= TOL * w.eps


LIMIT = {1: 2389, 2: 2389, 3: 2389, 4: 1433, 5: 1433, 6: 1433, 7: 1433, 8: 1024}


@pytest.mark.parametrize("d", [3, 7, 8])
def test_single_launch_at_size_limit(fs, d):
    n = (LIMIT[d] + 37) // 2
    w = workloads.random_cloud(700 + d, n, LIMIT[d] - n, d, weights="uniform",
                               scale=1.0 / np.sqrt(d))
    eps = 0.1
    f, g, info = _solve(w, eps, 3, 1)
    assert info["single_launch"]
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=eps, iters=3)
    assert max_err(f, ref["f"]) <= TOL * eps and max_err(g, ref["g"]) <= TOL * eps


@pytest.mark.parametrize("d", [1, 4, 8])
def test_single_launch_past_size_limit(fs, d):
    # one point more than the limit: the multi-launch path runs
    n = LIMIT[d] // 2
    w = workloads.random_cloud(800 + d, n, LIMIT[d] + 1 - n, d, weights="uniform",
                               scale=1.0 / np.sqrt(d))
    f, g, info = _solve(w, 0.2, 2, 1)
    assert not info["single_launch"] and info["lse_launches"] == 4
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=0.2, iters=2)
    assert max_err(f, ref["f"]) <= TOL * 0.2 and max_err(g, ref["g"]) <= TOL * 0.2


def test_single_launch_annealed_and_warm(fs):
    w = workloads.make("c5", n=700, m=600)
    f, g, info = _solve(w, w.eps, 4, 1, n_stages=5, eps_start=0.5)
    assert info["single_launch"]
    assert info["iters_done"] == 20 and abs(info["final_eps"] - w.eps) <= 1e-9
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=w.eps, eps_start=0.5, n_stages=5, iters=4)
    assert max_err(f, ref["f"]) <= TOL * w.eps and max_err(g, ref["g"]) <= TOL * w.eps
    # warm start from a given g
    g0 = np.random.default_rng(3).normal(0, 0.01, w.m)
    f, g, _ = _solve(w, 0.05, 6, 1, g0=g0)
    import oracle

    r = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=0.05, iters=6, g0=g0.astype(np.float32))
    assert max_err(f, r["f"]) <= TOL * 0.05 and max_err(g, r["g"]) <= TOL * 0.05


def test_single_launch_not_taken_when_not_allowed(fs):
    # too many points for the single launch: the multi-launch path runs
    w = workloads.random_cloud(5, 4000, 3600, 3, weights="uniform", scale=0.5)
    f, g, info = _solve(w, 0.2, 2, 1)
    assert not info["single_launch"] and info["lse_launches"] == 4 and np.all(np.isfinite(f))
    # by default only problems of at most 2^19 pairs take it, and never with a
    # residual stop
    w = workloads.random_cloud(6, 300, 200, 3, weights="uniform", scale=0.5)
    _, _, info = _solve(w, 0.2, 2, 0)
    assert info["single_launch"]
    import torch

    from streaming_sinkhorn_solver_amd import binding

    f, g = torch.empty(w.n, device="cuda"), torch.empty(w.m, device="cuda")
    p = binding.fs_potentials_init(dev(w.X), dev(w.Y), dev(w.a), dev(w.b), f=f, g=g)
    info = binding.fs_sinkhorn_solve(p, f, g, eps_end=0.2, iters_per_stage=50, tol=1e-4,
                                     check_every=5, single_launch=1, raise_not_converged=False)
    assert not info["single_launch"] and info["residual"] >= 0
    w = workloads.random_cloud(7, 1000, 1000, 2, weights="uniform", scale=0.5)
    _, _, info = _solve(w, 0.2, 2, 0)
    assert not info["single_launch"]  # 10^6 pairs > 2^19: not by default
    _, _, info = _solve(w, 0.2, 2, 1)
    assert info["single_launch"]


def test_single_launch_long_schedule(fs):
    # thousands of half-steps in one launch (every word tag distinct), against
    # the separate launches of the same schedule
    w = workloads.random_cloud(9, 400, 350, 2, weights="exp", scale=0.7)
    f, g, info = _solve(w, 0.05, 1500, 1, n_stages=3, eps_start=0.5)
    assert info["single_launch"] and info["iters_done"] == 4500
    f2, g2, _ = _solve(w, 0.05, 1500, -1, n_stages=3, eps_start=0.5)
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    assert max_err(f, f2) <= TOL * 0.05 and max_err(g, g2) <= TOL * 0.05
