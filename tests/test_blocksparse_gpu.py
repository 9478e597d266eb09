"""GPU parity of the block-sparse low-dimensional form (Morton order, block
screening, retained-block updates) against the oracle (oracle/blocksparse.py
and the dense oracle update).

* Morton order: bit-exact permutation (the codes are integer decisions taken
  in float32 on both sides, every step correctly rounded).
* Updates: the kept blocks are a choice the two sides make in different
  precisions (fp32 fits and bounds here, float64 in the oracle), so the
  lists are compared by what is unique: every block the GPU skips carries a
  true mass below delta / N_J of its rows' targets (brute force), and every
  block the oracle keeps with a margin is kept.  The potentials are then
  compared with the dense oracle update through the certificate,
      -tol <= f_gpu - f_dense <= eps log(1 + delta exp((f_gpu - f_cur)/eps)) + tol,
  with tol = 1e-3 eps, the fp32 parity bar of the dense path.
"""
import numpy as np
import pytest

import oracle
from oracle import blocksparse as obs
from helpers import dev, host

pytestmark = pytest.mark.gpu

TOL = 1e-3  # x eps


def _bind():
    from streaming_sinkhorn_solver_amd import binding as B
    return B


def _cloud(rng, n, d, kind):
    if kind == "uniform":
        return rng.uniform(0, 1, (n, d))
    if kind == "mixture":
        means = rng.uniform(0.2, 0.8, (8, d))
        return means[rng.integers(0, 8, n)] + rng.normal(0, 0.05, (n, d))
    if kind == "dups":
        base = rng.uniform(0, 1, (max(1, n // 7), d))
        return base[rng.integers(0, len(base), n)]
    raise ValueError(kind)


@pytest.mark.parametrize("n,d,kind", [(1, 3, "uniform"), (5, 1, "uniform"), (4095, 3, "uniform"),
                                      (4097, 2, "mixture"), (30001, 3, "dups"),
                                      (300_003, 3, "mixture"), (70_000, 1, "uniform"),
                                      (20_000, 8, "uniform")])
def test_morton_sort_bit_exact(n, d, kind):
    import torch

    B = _bind()
    rng = np.random.default_rng(n + d)
    X = _cloud(rng, n, d, kind).astype(np.float32)
    w = rng.standard_exponential(n).astype(np.float32)
    Xs, ws, perm = B.fs_morton_sort(dev(X), dev(w))
    torch.cuda.synchronize()
    ref = obs.morton_order(X)
    got = perm.cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(Xs.cpu().numpy(), X[ref])
    assert np.array_equal(ws.cpu().numpy(), w[ref])
    back = B.fs_unpermute(Xs, perm)
    assert np.array_equal(back.cpu().numpy(), X)


def _sorted_problem(seed, n, m, d, xkind="uniform", ykind="mixture"):
    rng = np.random.default_rng(seed)
    X = _cloud(rng, n, d, xkind)
    Y = _cloud(rng, m, d, ykind)
    X = X[obs.morton_order(X.astype(np.float32))].astype(np.float32)
    Y = Y[obs.morton_order(Y.astype(np.float32))].astype(np.float32)
    a = rng.standard_exponential(n)
    b = rng.standard_exponential(m)
    return X, Y, (a / a.sum()).astype(np.float32), (b / b.sum()).astype(np.float32)


def _gpu_problem(X, Y, a, b):
    B = _bind()
    p = B.fs_potentials_init(dev(X), dev(Y), dev(a), dev(b))
    B.fs_bs_attach(p)
    return p


def _check_lists(p, side, R, K, w_keys, pot_rows, pot_keys, eps, delta, chunk=0):
    """Every skipped block's true mass is below delta/N_J of its rows' targets;
    every block the oracle keeps with a margin is kept (with chunks: a block
    whose own and whose chunk's bounds clear the threshold by that margin)."""
    B = _bind()
    counts, L = B.fs_bs_read_screen(p, side, lists=True)
    nbR, nbK = len(counts), (len(K) + 31) // 32
    bounds = obs.screen(R, K, w_keys, pot_rows, pot_keys, eps, delta, 256, 32,
                        return_bounds=True, chunk=chunk)
    ref_lists, beta, thr = bounds[:3]
    if chunk:
        beta = np.where(np.repeat(bounds[3] >= thr + 1e-3, chunk, axis=1)[:, :nbK], beta, -np.inf)
    R64, K64 = R.astype(np.float64), K.astype(np.float64)
    skipped = 0
    for I in range(nbR):
        kept = L[I, :counts[I]]
        assert np.all(np.diff(kept) > 0) and kept.min() >= 0 and kept.max() < nbK
        pad = L[I, counts[I]:(counts[I] + 15) // 16 * 16]
        assert np.all(pad == (len(K) + 511) // 512 * 512 // 32)
        sure = np.nonzero(beta[I] >= thr + 1e-3)[0]
        assert set(sure.tolist()) <= set(kept.tolist())
        skip = np.setdiff1d(np.arange(nbK), kept)
        skipped += len(skip)
        if len(skip) == 0:
            continue
        rows = np.arange(I * 256, min((I + 1) * 256, len(R)))
        keys = np.concatenate([np.arange(J * 32, min(J * 32 + 32, len(K))) for J in skip])
        blk = np.concatenate([np.full(min(J * 32 + 32, len(K)) - J * 32, k)
                              for k, J in enumerate(skip)])
        C = ((R64[rows, None, :] - K64[None, keys, :]) ** 2).sum(-1)
        z = np.exp((pot_rows[rows, None] + pot_keys[None, keys] - C) / eps) * w_keys[None, keys]
        mass = np.zeros((len(rows), len(skip)))
        np.add.at(mass.T, blk, z.T)
        assert mass.max() < delta / nbK * 1.001
    return skipped / (nbR * nbK)


def _dense_converged(X, Y, a, b, eps, iters=400):
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=iters)
    return r["f"], r["g"]


# min_skip: the share of block pairs that must have been skipped (at these
# sizes a 256-row block spans a large part of the cloud, so it is small)
@pytest.mark.parametrize("n,m,d,eps,delta,min_skip", [(3000, 2500, 3, 2e-3, 1e-3, 0.02),
                                                      (1000, 4100, 2, 1e-3, 1e-4, 0.05),
                                                      (700, 900, 1, 1e-3, 1e-3, 0.05),
                                                      (200, 20, 3, 5e-3, 1e-3, 0.0)])
def test_bs_update_certificate(n, m, d, eps, delta, min_skip):
    import torch

    B = _bind()
    X, Y, a, b = _sorted_problem(n + m, n, m, d)
    f, g = _dense_converged(X, Y, a, b, eps, iters=150)
    p = _gpu_problem(X, Y, a, b)
    fd, gd = dev(f), dev(g)
    f_out = torch.empty_like(fd)
    B.fs_bs_lse_update_f(p, eps, delta, gd, fd, f_out)
    torch.cuda.synchronize()
    fs = host(f_out)
    frac_f = _check_lists(p, 0, X, Y, b.astype(np.float64), f, g, eps, delta)
    ref = oracle.f_update(X, Y, b, g, eps)
    cert = obs.certificate(fs, f, eps, delta)
    diff = fs - ref
    assert diff.min() >= -TOL * eps
    assert np.all(diff <= cert + TOL * eps)
    # the g side, from the new f
    g_out = torch.empty_like(gd)
    B.fs_bs_lse_update_g(p, eps, delta, f_out, gd, g_out)
    torch.cuda.synchronize()
    gs = host(g_out)
    frac_g = _check_lists(p, 1, Y, X, a.astype(np.float64), g, fs, eps, delta)
    ref = oracle.g_update(X, Y, a, fs, eps)
    cert = obs.certificate(gs, g, eps, delta)
    assert (gs - ref).min() >= -TOL * eps
    assert np.all(gs - ref <= cert + TOL * eps)
    print(f"skipped block pairs: f {frac_f:.3f}  g {frac_g:.3f}")
    assert frac_f >= min_skip and frac_g >= min_skip


@pytest.mark.parametrize("delta", [1e-3, 0.0])
def test_bs_two_level_screening(delta, monkeypatch):
    """With FS_BS_MIN_CHUNKS=4 a key cloud of 5 chunks of 8192 keys takes the
    two-level screening: the kept lists against the oracle's two-level screening
    (brute-force mass of every skipped block, every block kept by the oracle
    with a margin kept), on both sides, and the update within the
    certificate of the dense oracle update."""
    import torch

    B = _bind()
    n, m, eps = 1024, 33000, 2e-3
    X, Y, a, b = _sorted_problem(71, n, m, 3, xkind="mixture", ykind="uniform")
    # a consistent pair (f the exact update from g = 0: every row's mass sums
    # to its target), at which far blocks hold little mass
    g = np.zeros(m)
    f = oracle.f_update(X, Y, b, g, eps)
    monkeypatch.setenv("FS_BS_MIN_CHUNKS", "4")  # read by fs_bs_attach
    p = _gpu_problem(X, Y, a, b)
    f_new = torch.empty(n, device="cuda")
    B.fs_bs_lse_update_f(p, eps, delta, dev(g), dev(f), f_new)
    torch.cuda.synchronize()
    frac = _check_lists(p, 0, X, Y, b, f, g, eps, delta, chunk=256)
    if delta > 0:
        assert frac > 0.3
        counts, L = B.fs_bs_read_screen(p, 0, lists=True)
        nbC = (m + 8191) // 8192
        open_chunks = [set((L[I, :counts[I]] // 256).tolist()) for I in range(len(counts))]
        assert min(len(c) for c in open_chunks) < nbC  # whole chunks were skipped
    ref = oracle.f_update(X, Y, b, g, eps)
    fn = host(f_new)
    cert = obs.certificate(fn, f, eps, delta)
    assert np.all(fn - ref >= -TOL * eps) and np.all(fn - ref <= cert + TOL * eps)
    # the g side: keys X (1024 points, one-level form)
    g_new = torch.empty(m, device="cuda")
    B.fs_bs_lse_update_g(p, eps, delta, dev(f), dev(g), g_new)
    torch.cuda.synchronize()
    _check_lists(p, 1, Y, X, a, g, f, eps, delta)


def test_bs_delta_zero_is_the_dense_update():
    import torch

    B = _bind()
    X, Y, a, b = _sorted_problem(21, 1500, 1300, 3)
    rng = np.random.default_rng(22)
    eps = 0.01
    g = rng.normal(0, 0.01, 1300)
    f = rng.normal(0, 0.01, 1500)
    p = _gpu_problem(X, Y, a, b)
    out = torch.empty(1500, device="cuda")
    B.fs_bs_lse_update_f(p, eps, 0.0, dev(g), dev(f), out)
    counts = B.fs_bs_read_screen(p, 0)
    assert np.all(counts == (1300 + 31) // 32)
    ref = oracle.f_update(X, Y, b, g, eps)
    assert np.max(np.abs(host(out) - ref)) <= TOL * eps
    dense = torch.empty_like(out)
    B.fs_lse_update_f(p, eps, dev(g), dense)
    torch.cuda.synchronize()
    assert np.max(np.abs(host(out) - host(dense))) <= 1e-4 * eps


def _cert(new, cur, eps, delta):
    """eps log(1 + delta exp((new - cur)/eps)): the most a screened update can
    exceed the dense one when every skipped block holds below delta / N_J of
    each of its rows' targets ("FlashSinkhorn 2" explainer, guaranteeing the
    skip; the bound of the skipped mass at the current potentials)."""
    new, cur = np.asarray(new, np.float64), np.asarray(cur, np.float64)
    return eps * np.log1p(delta * np.exp((new - cur) / eps))


def test_bs_solve_fixed_iterations():
    """delta = 0: ten block-sparse iterations from zero equal the dense oracle
    iteration at the fp32 bar.  delta > 0: every half-step of three
    block-sparse iterations from a converged warm start is judged against the
    dense oracle update of the GPU's own inputs through the certificate (no
    reference takes a screening decision), and fs_bs_sinkhorn_solve over the
    same three iterations reproduces those half-steps bit for bit."""
    import torch

    B = _bind()
    X, Y, a, b = _sorted_problem(31, 1200, 1000, 3)
    eps, iters = 5e-3, 10
    p = _gpu_problem(X, Y, a, b)
    f = torch.zeros(1200, device="cuda")
    g = torch.zeros(1000, device="cuda")
    B.fs_bs_sinkhorn_solve(p, f, g, eps_end=eps, iters_per_stage=iters, delta=0.0)
    torch.cuda.synchronize()
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=iters)
    print(f"delta = 0: max|f - f_ref| {np.max(np.abs(host(f) - r['f'])) / eps:.2e} eps, "
          f"max|g - g_ref| {np.max(np.abs(host(g) - r['g'])) / eps:.2e} eps")
    assert np.max(np.abs(host(f) - r["f"])) <= TOL * eps
    assert np.max(np.abs(host(g) - r["g"])) <= TOL * eps
    delta = 1e-4
    fw, gw = _dense_converged(X, Y, a, b, eps, iters=200)
    f, g = dev(fw), dev(gw)
    for it in range(3):
        f_new = torch.empty_like(f)
        B.fs_bs_lse_update_f(p, eps, delta, g, f, f_new)
        torch.cuda.synchronize()
        fc, gc, fn = host(f), host(g), host(f_new)
        ref = oracle.f_update(X, Y, b, gc, eps)
        assert np.all(fn - ref >= -TOL * eps), (it, "f", np.min(fn - ref) / eps)
        assert np.all(fn - ref <= _cert(fn, fc, eps, delta) + TOL * eps), (it, "f")
        g_new = torch.empty_like(g)
        B.fs_bs_lse_update_g(p, eps, delta, f_new, g, g_new)
        torch.cuda.synchronize()
        gn = host(g_new)
        ref = oracle.g_update(X, Y, a, fn, eps)
        assert np.all(gn - ref >= -TOL * eps), (it, "g", np.min(gn - ref) / eps)
        assert np.all(gn - ref <= _cert(gn, gc, eps, delta) + TOL * eps), (it, "g")
        f, g = f_new, g_new
    fs_, gs_ = dev(fw), dev(gw)
    B.fs_bs_sinkhorn_solve(p, fs_, gs_, eps_end=eps, iters_per_stage=3, delta=delta,
                           warm_start=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(fs_), host(f)) and np.array_equal(host(gs_), host(g))


def test_bs_solve_residual_stop():
    import torch

    B = _bind()
    X, Y, a, b = _sorted_problem(41, 2000, 1800, 2)
    eps = 0.02
    p = _gpu_problem(X, Y, a, b)
    f = torch.zeros(2000, device="cuda")
    g = torch.zeros(1800, device="cuda")
    info = B.fs_bs_sinkhorn_solve(p, f, g, eps_end=eps, iters_per_stage=2000, delta=1e-5,
                                  tol=1e-3, check_every=5)
    assert info["residual"] <= 1e-3
    res = oracle.marginal_residual(X, Y, a, b, host(f), host(g), eps)
    assert res[0] + res[1] <= 2e-3


def test_bs_argument_errors():
    import torch

    B = _bind()
    rng = np.random.default_rng(51)
    X = rng.normal(size=(300, 4)).astype(np.float32)
    a = np.full(300, 1 / 300, np.float32)
    p4 = B.fs_potentials_init(dev(X), dev(X), dev(a), dev(a))
    assert B.fs_bs_workspace_bytes(p4) == 0
    with pytest.raises(B.FsError):
        B.fs_bs_attach(p4)
    X3 = X[:, :3].copy()
    pb = B.fs_potentials_init(dev(X3), dev(X3), dev(a), dev(a), prec="bf16")
    with pytest.raises(B.FsError):
        B.fs_bs_attach(pb)
    p3 = B.fs_potentials_init(dev(X3), dev(X3), dev(a), dev(a))
    f = torch.zeros(300, device="cuda")
    with pytest.raises(B.FsError):  # not attached
        B.fs_bs_lse_update_f(p3, 0.1, 1e-3, f, f, torch.empty_like(f))
    B.fs_bs_attach(p3)
    for delta in (-0.1, 1.0, float("nan")):
        with pytest.raises(B.FsError):
            B.fs_bs_lse_update_f(p3, 0.1, delta, f, f, torch.empty_like(f))
    with pytest.raises(B.FsError):  # residual with in-place output
        B.fs_bs_lse_update_f(p3, 0.1, 1e-3, f, f, f, row_resid=torch.empty(1, device="cuda"))
    with pytest.raises(B.FsError):
        B.fs_morton_sort(dev(np.zeros((10, 9), np.float32)))


@pytest.mark.parametrize("delta", [1e-3, 0.0])
def test_bs_transport(delta):
    """U = P.V over the kept blocks against the dense oracle transport:
    |U - U_dense| <= delta a_i max|V| (the skipped mass) + 2e-3 (P.|V|)_i
    (fp32), and the barycentric projection P.Y / a the same way."""
    import torch

    B = _bind()
    X, Y, a, b = _sorted_problem(61, 3000, 2500, 3)
    eps = 2e-3
    f, g = _dense_converged(X, Y, a, b, eps, iters=150)
    p = _gpu_problem(X, Y, a, b)
    rng = np.random.default_rng(62)
    V = rng.normal(size=(2500, 5)).astype(np.float32)
    U = torch.empty((3000, 5), device="cuda")
    B.fs_bs_apply_transport(p, eps, delta, dev(f), dev(g), dev(V), U)
    torch.cuda.synchronize()
    ref = oracle.transport(X, Y, a, b, f, g, V, eps)
    ref_abs = oracle.transport(X, Y, a, b, f, g, np.abs(V), eps)
    env = delta * a[:, None] * np.abs(V).max() + 2e-3 * ref_abs
    assert np.all(np.abs(host(U) - ref) <= env)
    # barycentric projection
    Ub = torch.empty((3000, 3), device="cuda")
    B.fs_bs_apply_transport(p, eps, delta, dev(f), dev(g), dev(Y), Ub, divide_by_a=True)
    torch.cuda.synchronize()
    refb = oracle.transport(X, Y, a, b, f, g, Y, eps, divide_by_a=True)
    refb_abs = oracle.transport(X, Y, a, b, f, g, np.abs(Y), eps, divide_by_a=True)
    envb = delta * np.abs(Y).max() + 2e-3 * refb_abs
    assert np.all(np.abs(host(Ub) - refb) <= envb)
    if delta > 0:
        counts = B.fs_bs_read_screen(p, 0)
        assert counts.sum() < len(counts) * ((2500 + 31) // 32)  # blocks were skipped


@pytest.mark.parametrize("delta", [1e-3, 0.0])
def test_bs_transport_t(delta):
    """The column side U_j = sum_i P_ij W_i over the g-side kept blocks against
    the dense oracle: |U - U_dense| <= delta b_j max|W| + 2e-3 (P^T.|W|)_j, and
    the column barycentric projection P^T.X / b the same way."""
    import torch

    B = _bind()
    X, Y, a, b = _sorted_problem(63, 2600, 3100, 3, xkind="mixture", ykind="uniform")
    eps = 2e-3
    f, g = _dense_converged(X, Y, a, b, eps, iters=150)
    p = _gpu_problem(X, Y, a, b)
    rng = np.random.default_rng(64)
    W = rng.normal(size=(2600, 4)).astype(np.float32)
    U = torch.empty((3100, 4), device="cuda")
    B.fs_bs_apply_transport_t(p, eps, delta, dev(f), dev(g), dev(W), U)
    torch.cuda.synchronize()
    ref = oracle.transport_t(X, Y, a, b, f, g, W, eps)
    ref_abs = oracle.transport_t(X, Y, a, b, f, g, np.abs(W), eps)
    env = delta * b[:, None] * np.abs(W).max() + 2e-3 * ref_abs
    assert np.all(np.abs(host(U) - ref) <= env)
    Ub = torch.empty((3100, 3), device="cuda")
    B.fs_bs_apply_transport_t(p, eps, delta, dev(f), dev(g), dev(X), Ub, divide_by_b=True)
    torch.cuda.synchronize()
    refb = oracle.transport_t(X, Y, a, b, f, g, X, eps, divide_by_b=True)
    refb_abs = oracle.transport_t(X, Y, a, b, f, g, np.abs(X), eps, divide_by_b=True)
    assert np.all(np.abs(host(Ub) - refb) <= delta * np.abs(X).max() + 2e-3 * refb_abs)
    if delta > 0:
        counts = B.fs_bs_read_screen(p, 1)
        assert counts.sum() < len(counts) * ((2600 + 31) // 32)
    with pytest.raises(B.FsError):  # more than 16 columns
        B.fs_bs_apply_transport_t(p, eps, delta, dev(f), dev(g),
                                  dev(np.zeros((2600, 17), np.float32)),
                                  torch.empty((3100, 17), device="cuda"))


@pytest.mark.parametrize("delta,d", [(1e-3, 3), (0.0, 3), (1e-3, 2), (1e-3, 1)])
def test_bs_gradient(delta, d):
    """grad_x_i = 2 sum_j P_ij (x_i - y_j) and grad_y over the kept blocks
    against the dense oracle gradient, per component within the skipped-mass
    bound 2 delta a_i max_j |x_ic - y_jc| plus 2e-3 of 2 sum_j P_ij |x_ic - y_jc|
    (the relative error of the fp32 plan entries) plus 1e-5 a_i for the fp32
    sums (the mirror for grad_y; bounds by brute force in float64)."""
    import torch

    B = _bind()
    n, m = 2800, 2300
    X, Y, a, b = _sorted_problem(65 + d, n, m, d)
    eps = 2e-3
    f, g = _dense_converged(X, Y, a, b, eps, iters=150)
    p = _gpu_problem(X, Y, a, b)
    gx = torch.empty((n, d), device="cuda")
    gy = torch.empty((m, d), device="cuda")
    B.fs_bs_gradient(p, eps, delta, dev(f), dev(g), gx, gy)
    torch.cuda.synchronize()
    rx, ry = oracle.gradient(X, Y, a, b, f, g, eps)
    X64, Y64 = X.astype(np.float64), Y.astype(np.float64)
    D = X64[:, None, :] - Y64[None, :, :]                       # n x m x d
    P = a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - (D ** 2).sum(-1)) / eps)
    absD = np.abs(D)
    env_x = (2 * delta * a[:, None] * absD.max(axis=1)
             + 2e-3 * 2 * np.einsum("ij,ijc->ic", P, absD) + 1e-5 * a[:, None])
    env_y = (2 * delta * b[:, None] * absD.max(axis=0)
             + 2e-3 * 2 * np.einsum("ij,ijc->jc", P, absD) + 1e-5 * b[:, None])
    ex, ey = np.abs(host(gx) - rx), np.abs(host(gy) - ry)
    print(f"d={d} delta={delta}: grad_x error {ex.max():.2e}, grad_y error {ey.max():.2e}")
    assert np.all(ex <= env_x)
    assert np.all(ey <= env_y)
    # one side alone gives the same values
    gx2 = torch.empty((n, d), device="cuda")
    B.fs_bs_gradient(p, eps, delta, dev(f), dev(g), grad_x=gx2)
    torch.cuda.synchronize()
    assert torch.equal(gx, gx2)
    with pytest.raises(B.FsError):  # an output on top of an input
        fdev = dev(np.zeros(n * d, np.float32))
        B.fs_bs_gradient(p, eps, delta, fdev[:n], dev(g), grad_x=fdev.view(n, d))
