"""GPU parity of the backward-pass operations: the column-side transport
P^T.W, the gradient of the dual with respect to the points, and the dual
value, against the float64 oracle on the same seeded inputs and the same GPU
potentials; and of the cosine cost (solve and gradient).

Bars:
  P^T.W          relative Frobenius error <= 1e-3 (the transport bar: f16
                 weights in (0, 1] and an f16 copy of W scaled by a power of
                 two, ~2^-11 per product, averaged);
  gradient       relative Frobenius error <= 1e-3 of the gradient itself;
  dual value     relative 1e-12 (fp64 sums of exact fp32 x fp32 products).
For the bf16/fp16 paths the reference is the plan of the problem the path
solves (rounded centred points, fp32 per-point cost terms; see
tests/helpers.py), applied to the original points.
"""
import numpy as np
import pytest

import oracle
from helpers import RoundedProblem, centres, dev, gpu_solve, host
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu


def _problem(prec, d, n, m):
    if prec in ("bf16", "fp16"):
        w = workloads.make("c3", n=n, m=m, d=d)
        return w.X, w.Y, w.a, w.b, w.eps
    w = workloads.random_cloud(300 + d, n, m, d, weights="exp", scale=1.0 / np.sqrt(d))
    return w.X, w.Y, w.a, w.b, 0.1


def _plan_products(X, Y, a, b, f, g, eps, prec, V, side):
    """sum_j P_ij V_j (side 'row', V: m x k) or sum_i P_ij V_i (side 'col')
    under the plan the path solves, in float64."""
    if prec in ("bf16", "fp16"):
        rp = RoundedProblem(X, Y, prec)
        ff, gg, Xo, Yo = f - rp.alpha, g - rp.beta, rp.Xr, rp.Yr
    else:
        ff, gg, Xo, Yo = f, g, X, Y
    if side == "row":
        return oracle.transport(Xo, Yo, a, b, ff, gg, V, eps)
    return oracle.transport_t(Xo, Yo, a, b, ff, gg, V, eps)


CASES = [("auto", 3, 900, 700), ("fp32-valu", 5, 600, 900), ("auto", 64, 1100, 800),
         ("bf16", 512, 700, 900), ("fp16", 256, 800, 700), ("fp16", 1024, 300, 500)]


@pytest.mark.parametrize("prec,d,n,m", CASES)
def test_column_transport(fs, prec, d, n, m):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, eps = _problem(prec, d, n, m)
    dv = 130
    W = np.random.default_rng(d + n).standard_normal((n, dv)).astype(np.float32)
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=6, prec=prec, dv_max=max(dv, d))
    U = torch.empty((m, dv), device="cuda")
    T = torch.empty((m, dv), device="cuda")
    Wd = dev(W)
    binding.fs_apply_transport_t(p, eps, f, g, Wd, U)
    binding.fs_apply_transport_t(p, eps, f, g, Wd, T, divide_by_b=True)
    torch.cuda.synchronize()
    ref = _plan_products(X, Y, a, b, host(f), host(g), eps, prec, W, "col")
    for got, want in ((host(U), ref), (host(T), ref / np.asarray(b, np.float64)[:, None])):
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert rel <= 1e-3, rel


@pytest.mark.parametrize("prec,d,n,m", CASES)
def test_gradient(fs, prec, d, n, m):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, eps = _problem(prec, d, n, m)
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=eps, iters=8, prec=prec, dv_max=d)
    gX = torch.empty((n, d), device="cuda")
    gY = torch.empty((m, d), device="cuda")
    binding.fs_gradient(p, eps, f, g, Xd, Yd, gX, gY)
    torch.cuda.synchronize()
    fh, gh = host(f), host(g)
    nu, mu = (c.astype(np.float64) for c in centres(X, Y))
    X64, Y64 = np.asarray(X, np.float64), np.asarray(Y, np.float64)
    for side, got, P_, Q_, c in (("row", host(gX), X64, Y64, mu), ("col", host(gY), Y64, X64, nu)):
        moved = _plan_products(X, Y, a, b, fh, gh, eps, prec, Q_ - c, side)
        mass = _plan_products(X, Y, a, b, fh, gh, eps, prec, np.ones((Q_.shape[0], 1)), side)
        want = 2.0 * (mass * (P_ - c) - moved)
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        print(f"{prec} d={d} {side}: relative error {rel:.2e} of the gradient")
        assert rel <= 1e-3
    if prec in ("auto", "fp32-valu"):
        # on the fp32 paths the definition itself, summed pair by pair
        gXo, gYo = oracle.gradient(X, Y, a, b, fh, gh, eps)
        assert np.linalg.norm(host(gX) - gXo) <= 1e-3 * np.linalg.norm(gXo)
        assert np.linalg.norm(host(gY) - gYo) <= 1e-3 * np.linalg.norm(gYo)


def test_gradient_needs_dv_max(fs):
    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b, eps = _problem("auto", 16, 300, 200)
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=eps, iters=2, dv_max=8)
    import torch

    gX = torch.empty((300, 16), device="cuda")
    with pytest.raises(binding.FsError):
        binding.fs_gradient(p, eps, f, g, Xd, Yd, gX, None)


@pytest.mark.parametrize("prec,d", [("auto", 3), ("bf16", 128)])
def test_dual_value(fs, prec, d):
    X, Y, a, b, eps = _problem(prec, d, 1500, 1300)
    from streaming_sinkhorn_solver_amd import binding

    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=5, prec=prec)
    v = float(binding.fs_dual_value(p, f, g).cpu()[0])
    want = float(np.asarray(a, np.float64) @ host(f) + np.asarray(b, np.float64) @ host(g))
    assert abs(v - want) <= 1e-12 * max(1.0, abs(want))
    # against the oracle: its dual objective after the same iterations (the
    # exponential term vanishes after a g-update, up to the fp32 weight sums),
    # within the potentials' bar times the total mass sum(a) + sum(b)
    from helpers import oracle_solve

    ref = oracle_solve(X, Y, a, b, eps=eps, iters=5)
    d_ref = oracle.dual_objective(X, Y, a, b, ref["f"], ref["g"], eps)
    bar = (1e-3 if prec == "auto" else 2e-2) * eps * 2.0
    print(f"{prec} d={d}: dual {v:.8f} vs oracle {d_ref:.8f} ({abs(v - d_ref) / eps:.2e} eps)")
    assert abs(v - d_ref) <= bar


def _back(P, Pn, G):
    """A gradient with respect to normalised points Pn = P/|P|, taken back to
    the raw points P: (G - Pn (Pn . G)) / |P| per row."""
    return (G - Pn * np.sum(Pn * G, axis=1, keepdims=True)) / np.linalg.norm(
        P, axis=1, keepdims=True)


@pytest.mark.parametrize("prec,d,n,m", [("auto", 3, 700, 900), ("auto", 64, 900, 600),
                                        ("bf16", 256, 600, 700)])
def test_cosine_cost(fs, prec, d, n, m):
    """C = 2 - 2 cos(x, y): potentials against the oracle on the normalised
    clouds (formed in float32 as the library does, see helpers), gradients
    against the chain rule through the normalisation (pinned by finite
    differences in test_oracle_gradient.py)."""
    import torch

    from helpers import max_err, normalise_rows, oracle_solve
    from streaming_sinkhorn_solver_amd import binding

    rng = np.random.default_rng(500 + d)
    X = (rng.standard_normal((n, d)) + 0.3).astype(np.float32)
    Y = (rng.standard_normal((m, d)) * 1.5 - 0.2).astype(np.float32)
    a = rng.standard_exponential(n)
    b = rng.standard_exponential(m)
    a, b = (a / a.sum()).astype(np.float32), (b / b.sum()).astype(np.float32)
    eps = 0.05
    p, f, g, _, (Xd, Yd, _, _) = gpu_solve(X, Y, a, b, eps=eps, iters=10, prec=prec,
                                           dv_max=d, cost="cosine")
    Xn, Yn = normalise_rows(X), normalise_rows(Y)
    fh, gh = host(f), host(g)
    if prec in ("bf16", "fp16"):
        ref = RoundedProblem(Xn, Yn, prec).solve(a, b, eps=eps, iters=10)
        tol = 2e-3
    else:
        ref = oracle_solve(Xn, Yn, a, b, eps=eps, iters=10)
        tol = 1e-3
    assert max_err(fh, ref["f"]) <= tol * eps and max_err(gh, ref["g"]) <= tol * eps
    gX = torch.empty((n, d), device="cuda")
    gY = torch.empty((m, d), device="cuda")
    binding.fs_gradient(p, eps, f, g, Xd, Yd, gX, gY)
    torch.cuda.synchronize()
    nu, mu = (c.astype(np.float64) for c in centres(Xn, Yn))
    Xn64, Yn64 = Xn.astype(np.float64), Yn.astype(np.float64)
    for side, got, P_, Pn, Qn, c in (("row", host(gX), X, Xn64, Yn64, mu),
                                     ("col", host(gY), Y, Yn64, Xn64, nu)):
        moved = _plan_products(Xn, Yn, a, b, fh, gh, eps, prec, Qn - c, side)
        mass = _plan_products(Xn, Yn, a, b, fh, gh, eps, prec, np.ones((Qn.shape[0], 1)), side)
        want = _back(np.asarray(P_, np.float64), Pn, 2.0 * (mass * (Pn - c) - moved))
        bar = 1e-3 * 2.0 * np.linalg.norm(moved) / np.min(np.linalg.norm(P_, axis=1))
        err = np.linalg.norm(got - want)
        print(f"cosine {prec} d={d} {side}: error {err / bar * 1e-3:.2e} of the bar's scale, "
              f"{err / np.linalg.norm(want):.2e} of the gradient")
        assert err <= bar
        # the cosine cost ignores the points' lengths: grad . p = 0 per row
        assert np.max(np.abs(np.sum(got * P_, axis=1))) <= 1e-4 * np.max(np.abs(got)) * \
            np.max(np.linalg.norm(P_, axis=1))


def test_cosine_rejects_zero_length_points(fs):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    X = np.random.default_rng(0).standard_normal((100, 8)).astype(np.float32)
    X[17] = 0.0
    Y = np.random.default_rng(1).standard_normal((90, 8)).astype(np.float32)
    a = np.full(100, 0.01, np.float32)
    b = np.full(90, 1 / 90, np.float32)
    with pytest.raises(binding.FsError) as e:
        binding.fs_potentials_init(dev(X), dev(Y), dev(a), dev(b), cost="cosine")
    assert e.value.status == binding.FS_ERR_INVALID_ARG
    # the same points under the squared-Euclidean cost are fine
    binding.fs_potentials_init(dev(X), dev(Y), dev(a), dev(b))
    torch.cuda.synchronize()
