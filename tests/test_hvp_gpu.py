"""GPU parity of the streaming Hessian-vector product (fs_hvp) against the
dense float64 oracle (oracle/hvp.py, pinned in test_oracle_hvp.py) on the same
seeded inputs and the same GPU potentials.

The reference plan is the one the path solves: the original points for the
fp32 paths; for bf16/fp16 the rounded centred clouds with fp32 cost terms
(tests/helpers.py), with the cost derivative 2 (x_i - y_j).v_i taken from the
original points as the library does.  Bar: relative Frobenius error 2e-3
(5e-3 on the bf16 path).  Every term of the product comes from transports
whose f16 weights (in (0, 1], 2^-11 relative) and f16 copies of their inputs
(scaled by a power of two, 2^-11 relative) carry about 1e-3 relative error
per product, averaged down over the keys; the CG solve for dg stops at a
residual of 1e-4 of its start.  On the two-byte paths at d_pad 64..512 the
second-moment term comes from one pass whose direction scores v_i.y~_j
multiply copies of v and of the centred keys in the score type: bf16 keeps 8
significant bits (2^-9 relative per element, against fp16's 2^-11), which
moves that term by up to a few 1e-3 where few coordinates average it.
Observed: 2e-6 (fp32 vector paths), 1-2e-4 (fp16), 5.7e-4 (bf16, d = 512),
1.9e-3 (bf16, d = 64).
"""
import numpy as np
import pytest

from helpers import RoundedProblem, dev, gpu_solve, host
from oracle.hvp import hvp as oracle_hvp
from oracle.hvp import plan as oracle_plan
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu

# two-byte paths at d_pad 64..512 take the one-pass second-moment kernel
# (every row width it is built for); the others the d*d-column passes
CASES = [("auto", 3, 300, 250, 0.3), ("fp32-valu", 3, 200, 260, 0.5), ("auto", 16, 400, 350, 0.2),
         ("bf16", 64, 300, 280, None), ("fp16", 128, 260, 300, None),
         ("fp16", 256, 330, 270, None), ("bf16", 512, 250, 300, None), ("fp16", 1024, 70, 90, None)]


def _problem(prec, d, n, m):
    if prec in ("bf16", "fp16"):
        w = workloads.make("c3", n=n, m=m, d=d)
        return w.X, w.Y, w.a, w.b, w.eps
    rng = np.random.default_rng(40 + d + n)
    X = (rng.standard_normal((n, d)) / np.sqrt(d)).astype(np.float32)
    Y = (rng.standard_normal((m, d)) * 0.7 / np.sqrt(d) + 0.2 / np.sqrt(d)).astype(np.float32)
    a = rng.standard_exponential(n)
    b = rng.standard_exponential(m)
    return X, Y, (a / a.sum()).astype(np.float32), (b / b.sum()).astype(np.float32), None


def _reference(X, Y, a, b, f, g, V, eps, prec, wrt="x"):
    if prec in ("bf16", "fp16"):
        rp = RoundedProblem(X, Y, prec)
        P = oracle_plan(rp.Xr, rp.Yr, a, b, f - rp.alpha, g - rp.beta, eps)
        if wrt == "y":  # the same loss with the clouds exchanged: the plan transposed
            return oracle_hvp(Y, X, b, a, g, f, V, eps, P=P.T)
        return oracle_hvp(X, Y, a, b, f, g, V, eps, P=P)
    if wrt == "y":
        return oracle_hvp(Y, X, b, a, g, f, V, eps)
    return oracle_hvp(X, Y, a, b, f, g, V, eps)


@pytest.mark.parametrize("prec,d,n,m,eps", CASES)
def test_hvp_matches_oracle(fs, prec, d, n, m, eps):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, weps = _problem(prec, d, n, m)
    eps = eps or weps
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=eps, iters=40, prec=prec,
                                           dv_max=max(d + 2, min(d * d, 4096)))
    V = np.random.default_rng(d + n).standard_normal((n, d)).astype(np.float32)
    HV = torch.empty((n, d), device="cuda")
    info = binding.fs_hvp(p, eps, f, g, Xd, Yd, dev(V), HV, cg_tol=1e-4, cg_max_iter=300)
    torch.cuda.synchronize()
    ref = _reference(X, Y, a, b, host(f), host(g), V, eps, prec)
    got = host(HV)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"{prec} d={d}: HVP relative error {rel:.2e}, CG {info}")
    assert info["cg_residual"] <= 1e-4
    assert rel <= (5e-3 if prec == "bf16" else 2e-3)


@pytest.mark.parametrize("prec,d,n,m,eps", [CASES[0], CASES[2], CASES[3], CASES[4]])
def test_hvp_with_respect_to_y(fs, prec, d, n, m, eps):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, weps = _problem(prec, d, n, m)
    eps = eps or weps
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=eps, iters=40, prec=prec,
                                           dv_max=max(d + 2, min(d * d, 4096)))
    V = np.random.default_rng(d + m).standard_normal((m, d)).astype(np.float32)
    HV = torch.empty((m, d), device="cuda")
    info = binding.fs_hvp(p, eps, f, g, Xd, Yd, dev(V), HV, wrt="y")
    torch.cuda.synchronize()
    ref = _reference(X, Y, a, b, host(f), host(g), V, eps, prec, wrt="y")
    rel = np.linalg.norm(host(HV) - ref) / np.linalg.norm(ref)
    print(f"{prec} d={d} wrt y: HVP relative error {rel:.2e}, CG {info}")
    assert rel <= (5e-3 if prec == "bf16" else 2e-3)


def test_hvp_is_symmetric(fs):
    # <U, H V> = <V, H U> at any size (the Hessian of a scalar function)
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, _ = _problem("auto", 8, 2000, 1500)
    eps = 0.2
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=eps, iters=60, dv_max=64)
    rng = np.random.default_rng(9)
    U, V = (rng.standard_normal((2000, 8)).astype(np.float32) for _ in range(2))
    HU, HV = torch.empty((2000, 8), device="cuda"), torch.empty((2000, 8), device="cuda")
    binding.fs_hvp(p, eps, f, g, Xd, Yd, dev(U), HU, cg_tol=1e-5)
    binding.fs_hvp(p, eps, f, g, Xd, Yd, dev(V), HV, cg_tol=1e-5)
    torch.cuda.synchronize()
    lhs = float(np.sum(U.astype(np.float64) * host(HV)))
    rhs = float(np.sum(V.astype(np.float64) * host(HU)))
    print(f"symmetry: {lhs:.6e} vs {rhs:.6e}")
    assert abs(lhs - rhs) <= 2e-3 * max(abs(lhs), abs(rhs)), (lhs, rhs)


def test_hvp_argument_checks(fs):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, _ = _problem("auto", 8, 300, 200)
    V = torch.zeros((300, 8), device="cuda")
    HV = torch.empty((300, 8), device="cuda")
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=0.3, iters=3, dv_max=9)
    with pytest.raises(binding.FsError) as e:  # dv_max < d + 2
        binding.fs_hvp(p, 0.3, f, g, Xd, Yd, V, HV)
    assert e.value.status == binding.FS_ERR_INVALID_ARG
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=0.3, iters=3, dv_max=10)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.FsError) as e:
        binding.fs_hvp(p, 0.3, f, g, Xd, Yd, V, HV, workspace=small)
    assert e.value.status == binding.FS_ERR_WORKSPACE
    with pytest.raises(binding.FsError) as e:  # HV aliasing V
        binding.fs_hvp(p, 0.3, f, g, Xd, Yd, V, V)
    assert e.value.status == binding.FS_ERR_INVALID_ARG
    # a zero direction gives a zero product without CG work
    info = binding.fs_hvp(p, 0.3, f, g, Xd, Yd, V, HV)
    torch.cuda.synchronize()
    assert info["cg_iters"] == 0 and float(torch.max(torch.abs(HV))) == 0.0
