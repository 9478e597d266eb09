"""FS_PREC_BF16_REFINE: bf16 iterations with the last refine_iters
iterations and the passes at given potentials on fp16 copies of the same
centred points.

* Composition, bit for bit: a refined solve of K iterations equals K - r
  iterations of a bf16 problem followed by r iterations of an fp16 problem on
  the same inputs (r = refine_iters, default 1; annealed schedules too, with r
  a whole last stage or more); its transport, gradient and residual equal the
  fp16 problem's at the same potentials; with a residual stop, r fp16
  iterations follow the stop.
* Parity with the float64 oracle on the 512-D two-mixture recipe at a small
  size: potentials within 2e-2 eps and the barycentric projection within
  1e-3 relative of the oracle's, both after the same iterations.
* d <= 8 is rejected; the workspace holds the second operand copy.
"""
import numpy as np
import pytest

import oracle
from helpers import dev, host, max_err, oracle_solve
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu


def _pair(w, dv):
    """A refined problem and the two plain ones it stands for."""
    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b = dev(w.X), dev(w.Y), dev(w.a), dev(w.b)
    pr = binding.fs_potentials_init(X, Y, a, b, prec="bf16-refine", dv_max=dv)
    pb = binding.fs_potentials_init(X, Y, a, b, prec="bf16", dv_max=dv)
    ph = binding.fs_potentials_init(X, Y, a, b, prec="fp16", dv_max=dv)
    return pr, pb, ph, (X, Y, a, b)


def _split_schedule(binding, pb, ph, f, g, w, stages, iters, refine):
    """The schedule with its first stages*iters - refine iterations on the bf16
    problem and the rest on the fp16 problem, stage by stage."""
    import math

    e0 = w.eps_start if stages > 1 else w.eps
    a0, a1 = float(np.float32(e0)), float(np.float32(w.eps))
    t0 = stages * iters - refine
    started = False
    for s in range(stages):
        e = a1 if stages == 1 else float(np.float32(a0 * math.pow(a1 / a0, s / (stages - 1))))
        lo, hi = s * iters, (s + 1) * iters
        for p, k in ((pb, max(0, min(hi, t0) - lo)), (ph, max(0, hi - max(lo, t0)))):
            if k:
                binding.fs_sinkhorn_solve(p, f, g, eps_end=e, iters_per_stage=k,
                                          warm_start=started)
                started = True


@pytest.mark.parametrize("name,n,m,d,iters,stages,refine", [("c3", 1100, 900, 512, 12, 1, 0),
                                                            ("c3", 1100, 900, 512, 12, 1, 3),
                                                            ("c4", 700, 600, 1024, 3, 4, 0),
                                                            ("c4", 700, 600, 1024, 3, 4, 3),
                                                            ("c4", 700, 600, 1024, 3, 4, 5),
                                                            ("c2", 1500, 1300, 64, 20, 1, 0)])
def test_refined_solve_composes(fs, name, n, m, d, iters, stages, refine):
    """refine = 0 (one fp16 iteration), a whole last stage (c4: 3), or more
    than a stage (c4: 5, across the stage boundary)."""
    import torch

    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make(name, n=n, m=m, d=d)
    e0 = w.eps_start if stages > 1 else None
    pr, pb, ph, (X, Y, _, _) = _pair(w, max(d, 70))
    assert pr.info["path"] == "bf16-mfma-fp16-refine"
    f1, g1 = torch.empty(n, device="cuda"), torch.empty(m, device="cuda")
    info = binding.fs_sinkhorn_solve(pr, f1, g1, eps_end=w.eps, eps_start=e0, n_stages=stages,
                                     iters_per_stage=iters, refine_iters=refine)
    assert info["iters_done"] == stages * iters
    # the same schedule: all but the last max(refine, 1) iterations in bf16,
    # those in fp16
    f2, g2 = torch.empty(n, device="cuda"), torch.empty(m, device="cuda")
    _split_schedule(binding, pb, ph, f2, g2, w, stages, iters, max(refine, 1))
    torch.cuda.synchronize()
    assert np.array_equal(host(f1), host(f2)) and np.array_equal(host(g1), host(g2))
    # passes at given potentials run on the fp16 copies
    Vd = dev(np.random.default_rng(d).standard_normal((m, 70)).astype(np.float32))
    Ur, Uh = torch.empty((n, 70), device="cuda"), torch.empty((n, 70), device="cuda")
    binding.fs_apply_transport(pr, w.eps, f1, g1, Vd, Ur, divide_by_a=True)
    binding.fs_apply_transport(ph, w.eps, f1, g1, Vd, Uh, divide_by_a=True)
    gr = [torch.empty((n, d), device="cuda"), torch.empty((m, d), device="cuda")]
    gh = [torch.empty((n, d), device="cuda"), torch.empty((m, d), device="cuda")]
    binding.fs_gradient(pr, w.eps, f1, g1, X, Y, *gr)
    binding.fs_gradient(ph, w.eps, f1, g1, X, Y, *gh)
    rr, rh = torch.empty(2, device="cuda"), torch.empty(2, device="cuda")
    binding.fs_marginal_residual(pr, w.eps, f1, g1, rr)
    binding.fs_marginal_residual(ph, w.eps, f1, g1, rh)
    torch.cuda.synchronize()
    assert np.array_equal(host(Ur), host(Uh))
    assert np.array_equal(host(gr[0]), host(gh[0])) and np.array_equal(host(gr[1]), host(gh[1]))
    assert np.array_equal(host(rr), host(rh))
    # and the single updates stay bf16
    fr, fb = torch.empty_like(f1), torch.empty_like(f1)
    binding.fs_lse_update_f(pr, w.eps, g1, fr)
    binding.fs_lse_update_f(pb, w.eps, g1, fb)
    torch.cuda.synchronize()
    assert np.array_equal(host(fr), host(fb))


def test_refined_parity_against_oracle(fs):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make("c3", n=1000, m=900, d=512)
    iters = 10
    X, Y, a, b = dev(w.X), dev(w.Y), dev(w.a), dev(w.b)
    f, g = torch.empty(w.n, device="cuda"), torch.empty(w.m, device="cuda")
    p = binding.fs_potentials_init(X, Y, a, b, prec="bf16-refine", dv_max=w.d, f=f, g=g)
    binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=iters)
    T = torch.empty((w.n, w.d), device="cuda")
    binding.fs_apply_transport(p, w.eps, f, g, dev(w.Y), T, divide_by_a=True)
    torch.cuda.synchronize()
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=w.eps, iters=iters)
    ef, eg = max_err(host(f), ref["f"]) / w.eps, max_err(host(g), ref["g"]) / w.eps
    T_ref = oracle.transport(w.X, w.Y, w.a, w.b, ref["f"], ref["g"], w.Y, w.eps,
                             divide_by_a=True)
    rel = np.linalg.norm(host(T) - T_ref) / np.linalg.norm(T_ref)
    print(f"refined: f {ef:.2e} eps, g {eg:.2e} eps, P.Y/a rel {rel:.2e}")
    assert ef <= 2e-2 and eg <= 2e-2
    assert rel <= 1e-3


def test_refined_residual_stop(fs):
    """With a residual stop the checks measure the bf16 iteration and one fp16
    iteration follows the stop: bit for bit the bf16 problem's residual-stop
    solve plus one iteration of the fp16 problem."""
    import torch

    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make("c2", n=1200, m=1000, d=64)
    pr, pb, ph, _ = _pair(w, 0)
    f1, g1 = torch.empty(w.n, device="cuda"), torch.empty(w.m, device="cuda")
    info = binding.fs_sinkhorn_solve(pr, f1, g1, eps_end=w.eps, iters_per_stage=400, tol=1e-3,
                                     check_every=5)
    f2, g2 = torch.empty(w.n, device="cuda"), torch.empty(w.m, device="cuda")
    info_b = binding.fs_sinkhorn_solve(pb, f2, g2, eps_end=w.eps, iters_per_stage=400,
                                       tol=1e-3, check_every=5)
    binding.fs_sinkhorn_solve(ph, f2, g2, eps_end=w.eps, iters_per_stage=1, warm_start=True)
    torch.cuda.synchronize()
    assert info["iters_done"] == info_b["iters_done"] + 1 and info["iters_done"] % 5 == 1
    assert info["residual"] == info_b["residual"] and info["residual"] <= 1e-3
    assert np.array_equal(host(f1), host(f2)) and np.array_equal(host(g1), host(g2))
    # refine_iters fp16 iterations after the stop
    f3, g3 = torch.empty(w.n, device="cuda"), torch.empty(w.m, device="cuda")
    info3 = binding.fs_sinkhorn_solve(pr, f3, g3, eps_end=w.eps, iters_per_stage=400, tol=1e-3,
                                      check_every=5, refine_iters=3)
    binding.fs_sinkhorn_solve(ph, f2, g2, eps_end=w.eps, iters_per_stage=2, warm_start=True)
    torch.cuda.synchronize()
    assert info3["iters_done"] == info_b["iters_done"] + 3
    assert np.array_equal(host(f3), host(f2)) and np.array_equal(host(g3), host(g2))
    with pytest.raises(binding.FsError) as e:
        binding.fs_sinkhorn_solve(pr, f3, g3, eps_end=w.eps, iters_per_stage=4, refine_iters=-1)
    assert e.value.status == binding.FS_ERR_INVALID_ARG


def test_refined_rejects_small_d_and_doubles_operands(fs):
    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make("c1", n=100, m=90)
    with pytest.raises(binding.FsError) as e:
        binding.fs_potentials_init(dev(w.X), dev(w.Y), dev(w.a), dev(w.b), prec="bf16-refine")
    assert e.value.status == binding.FS_ERR_INVALID_ARG
    n, m, d = 20_000, 10_000, 512
    extra = binding.fs_workspace_bytes(n, m, d, 0, "bf16-refine") - \
        binding.fs_workspace_bytes(n, m, d, 0, "bf16")
    assert extra >= (20_480 + 10_240) * d * 2
