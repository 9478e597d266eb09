"""GPU parity of the coarse (centroid) stage against oracle/coarse.py:
centroids (1e-6 relative: fp64 sums rounded to fp32), the lift (exact), the
sampled marginal check (1e-4 relative, plus 1e-6 absolute: an fp32 LSE over
the other cloud), and the whole coarse start (rounds and acceptance equal,
lifted potentials within the fp32 parity bar 1e-3 eps of the oracle's)."""
import numpy as np
import pytest

import oracle
from oracle import blocksparse as obs
from oracle import coarse as oc
from helpers import dev, host

pytestmark = pytest.mark.gpu


def _bind():
    from streaming_sinkhorn_solver_amd import binding as B
    return B


def _pair(seed, n, m, d=3):
    rng = np.random.default_rng(seed)
    X = rng.uniform(0, 1, (n, d))
    Y = rng.uniform(0, 1, (m, d)) * 0.9 + 0.05
    X = X[obs.morton_order(X.astype(np.float32))].astype(np.float32)
    Y = Y[obs.morton_order(Y.astype(np.float32))].astype(np.float32)
    a, b = rng.standard_exponential(n), rng.standard_exponential(m)
    return X, Y, (a / a.sum()).astype(np.float32), (b / b.sum()).astype(np.float32)


@pytest.mark.parametrize("n,d,cell", [(1, 3, 4), (257, 1, 7), (5000, 3, 64), (4099, 8, 1),
                                      (100_003, 2, 16)])
def test_centroids_and_lift(n, d, cell):
    import torch

    B = _bind()
    rng = np.random.default_rng(n + d)
    P = rng.normal(size=(n, d)).astype(np.float32)
    w = rng.standard_exponential(n).astype(np.float32)
    C, W = B.fs_centroids(dev(P), dev(w), cell)
    torch.cuda.synchronize()
    Cr, Wr = oc.centroids(P, w, cell)
    np.testing.assert_allclose(host(W), Wr, rtol=1e-6)
    np.testing.assert_allclose(host(C), Cr, rtol=1e-6, atol=1e-6)
    F = rng.normal(size=len(Wr)).astype(np.float32)
    f = B.fs_lift(dev(F), n, cell)
    torch.cuda.synchronize()
    assert np.array_equal(host(f), oc.lift(F, n, cell))


def test_sampled_marginal_error():
    import torch

    B = _bind()
    X, Y, a, b = _pair(7, 3000, 2500)
    rng = np.random.default_rng(8)
    eps = 0.02
    f = rng.normal(0, 0.01, 3000).astype(np.float32)
    g = rng.normal(0, 0.01, 2500).astype(np.float32)
    rows = np.sort(rng.choice(3000, 300, replace=False)).astype(np.int32)
    cols = np.sort(rng.choice(2500, 200, replace=False)).astype(np.int32)
    out = B.fs_sampled_marginal_error(dev(X), dev(Y), dev(a), dev(b), dev(f), dev(g), eps,
                                      torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda())
    torch.cuda.synchronize()
    ref = oc.sampled_marginal_error(X, Y, a, b, f, g, eps, rows, cols)
    np.testing.assert_allclose(host(out), ref, rtol=1e-4, atol=1e-6)
    # every row and column: the full L1 residual
    allr = torch.arange(3000, dtype=torch.int32, device="cuda")
    allc = torch.arange(2500, dtype=torch.int32, device="cuda")
    out = B.fs_sampled_marginal_error(dev(X), dev(Y), dev(a), dev(b), dev(f), dev(g), eps, allr,
                                      allc)
    full = oracle.marginal_residual(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(host(out), [full[1], full[2]], rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("cell,tol,rounds", [(4, 0.3, 1), (4, 1e-9, 3)])
def test_coarse_start(cell, tol, rounds):
    import torch

    B = _bind()
    X, Y, a, b = _pair(4, 800, 700)
    rng = np.random.default_rng(5)
    rows = rng.choice(800, 64, replace=False).astype(np.int32)
    cols = rng.choice(700, 64, replace=False).astype(np.int32)
    eps = 0.05
    ref = oc.coarse_start(X, Y, a, b, cell, eps, 30, n_stages=4, eps_start=0.2, more_iters=20,
                          tol=tol, max_rounds=3, rows=rows, cols=cols)
    Xd, Yd, ad, bd = dev(X), dev(Y), dev(a), dev(b)
    CX, WX = B.fs_centroids(Xd, ad, cell)
    CY, WY = B.fs_centroids(Yd, bd, cell)
    F = torch.empty(CX.shape[0], device="cuda")
    G = torch.empty(CY.shape[0], device="cuda")
    pc = B.fs_potentials_init(CX, CY, WX, WY, f=F, g=G)
    f = torch.empty(800, device="cuda")
    g = torch.empty(700, device="cuda")
    info = B.fs_bs_coarse_start(pc, Xd, Yd, ad, bd, cell, f, g, F, G,
                                torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda(),
                                eps_end=eps, iters_per_stage=30, n_stages=4, eps_start=0.2,
                                more_iters=20, check_tol=tol, max_rounds=3)
    torch.cuda.synchronize()
    assert info["rounds"] == ref["rounds"] == rounds
    assert info["accepted"] == ref["accepted"]
    assert np.max(np.abs(host(f) - ref["f"])) <= 1e-3 * eps
    assert np.max(np.abs(host(g) - ref["g"])) <= 1e-3 * eps
    np.testing.assert_allclose([info["err_rows"], info["err_cols"]], ref["errors"], rtol=2e-3)


def test_coarse_start_block_sparse():
    """The coarse stage with its coarse solves in block-sparse form: the coarse
    potentials equal those of fs_bs_sinkhorn_solve run with the same schedule
    and delta on the same coarse problem (bit for bit: same launches, and that
    solve has its own parity tests against the oracle's sparse iteration), the
    lift copies them exactly, and the check's errors match the oracle's
    sampled check on the lifted potentials (1e-4 relative)."""
    import torch

    B = _bind()
    n, m, cell = 24000, 20000, 4
    X, Y, a, b = _pair(14, n, m)
    rng = np.random.default_rng(15)
    rows = rng.choice(n, 128, replace=False).astype(np.int32)
    cols = rng.choice(m, 128, replace=False).astype(np.int32)
    eps, delta = 2e-3, 1e-3
    Xd, Yd, ad, bd = dev(X), dev(Y), dev(a), dev(b)
    CX, WX = B.fs_centroids(Xd, ad, cell)
    CY, WY = B.fs_centroids(Yd, bd, cell)
    F = torch.empty(CX.shape[0], device="cuda")
    G = torch.empty(CY.shape[0], device="cuda")
    pc = B.fs_potentials_init(CX, CY, WX, WY, f=F, g=G)
    with pytest.raises(B.FsError):  # not attached
        B.fs_bs_coarse_start(pc, Xd, Yd, ad, bd, cell, torch.empty(n, device="cuda"),
                             torch.empty(m, device="cuda"), F, G, torch.from_numpy(rows).cuda(),
                             torch.from_numpy(cols).cuda(), eps_end=eps, iters_per_stage=5,
                             coarse_delta=delta)
    B.fs_bs_attach(pc)
    f = torch.empty(n, device="cuda")
    g = torch.empty(m, device="cuda")
    sched = dict(eps_end=eps, iters_per_stage=10, n_stages=6, eps_start=0.1)
    info = B.fs_bs_coarse_start(pc, Xd, Yd, ad, bd, cell, f, g, F, G,
                                torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda(),
                                more_iters=0, check_tol=1e-9, max_rounds=1, coarse_delta=delta,
                                **sched)
    F2 = torch.zeros_like(F)
    G2 = torch.zeros_like(G)
    B.fs_bs_sinkhorn_solve(pc, F2, G2, delta=delta, **sched)
    torch.cuda.synchronize()
    assert torch.equal(F, F2) and torch.equal(G, G2)
    counts = B.fs_bs_read_screen(pc, 1)
    sh = B.fs_bs_shape(pc, 1)
    assert counts.sum() < sh["row_blocks"] * sh["key_blocks"]  # the coarse solve skipped blocks
    fh, gh = host(f), host(g)
    assert np.array_equal(fh, host(F)[np.arange(n) // cell])
    assert np.array_equal(gh, host(G)[np.arange(m) // cell])
    ref = oc.sampled_marginal_error(X, Y, a, b, fh, gh, eps, rows, cols)
    np.testing.assert_allclose([info["err_rows"], info["err_cols"]], ref, rtol=1e-4)
    assert info["rounds"] == 1 and not info["accepted"]


def test_coarse_argument_errors():
    import torch

    B = _bind()
    X, Y, a, b = _pair(9, 100, 90)
    Xd, ad = dev(X), dev(a)
    with pytest.raises(B.FsError):
        B.fs_centroids(Xd, ad, 0)
    CX, WX = B.fs_centroids(Xd, ad, 8)
    CY, WY = B.fs_centroids(dev(Y), dev(b), 8)
    pc = B.fs_potentials_init(CX, CY, WX, WY)
    f, g = torch.empty(100, device="cuda"), torch.empty(90, device="cuda")
    F, G = torch.empty(pc.n, device="cuda"), torch.empty(pc.m, device="cuda")
    r = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(B.FsError):  # cell does not match the coarse problem
        B.fs_bs_coarse_start(pc, Xd, dev(Y), ad, dev(b), 4, f, g, F, G, r, r, eps_end=0.1,
                             iters_per_stage=5)
