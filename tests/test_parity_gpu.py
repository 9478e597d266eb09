"""GPU parity: the HIP solver against the float64 oracle, same seeded inputs,
same fixed iteration count, element by element.

Tolerances (on every potential entry, after the same number of iterations):
  fp32 score paths       max|f - f_ref|, max|g - g_ref| <= 1e-3 eps
  bf16/fp16 score paths  <= 2e-2 eps against the oracle on the original
                         points, and <= 2e-3 eps against the oracle run on the
                         problem the path actually solves (the rounded
                         centred points plus the fp32 per-point cost terms;
                         isolates kernel error from quantisation)
  transport              ||U - U_ref||_F / ||U_ref||_F <= 1e-3
Sizes span several tiles and splits with ragged tails; the oracle finishes
each case in seconds.
"""
import numpy as np
import pytest

import oracle
from helpers import RoundedProblem, dev, gpu_solve, host, max_err, oracle_solve
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu

TOL_FP32 = 1e-3
TOL_LOWP = 2e-2
TOL_LOWP_ROUNDED = 2e-3


def _problem(seed, n, m, d, weights="exp", scale=1.0):
    w = workloads.random_cloud(seed, n, m, d, weights=weights, scale=scale)
    return w.X, w.Y, w.a, w.b


def test_c1_full_against_stored_oracle(fs):
    import os

    w = workloads.make("c1")
    _, f, g, _, _ = gpu_solve(w.X, w.Y, w.a, w.b, eps=w.eps, iters=w.iters)
    gold = os.path.join(os.path.dirname(__file__), "golden")
    f_ref = np.loadtxt(os.path.join(gold, "c1_oracle_f_iter100.txt"))
    g_ref = np.loadtxt(os.path.join(gold, "c1_oracle_g_iter100.txt"))
    assert max_err(host(f), f_ref) <= TOL_FP32 * w.eps
    assert max_err(host(g), g_ref) <= TOL_FP32 * w.eps


SMALL_D_PATHS = [("auto", "fp32-small-mfma"), ("fp32-valu", "fp32-valu")]


@pytest.mark.parametrize("prec,path", SMALL_D_PATHS)
@pytest.mark.parametrize("d", [1, 2, 3, 4, 5, 6, 7, 8])
def test_small_d_paths_ragged(fs, prec, path, d):
    X, Y, a, b = _problem(100 + d, 1000 + 37 * d, 777, d)
    eps = 0.2
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=15, prec=prec)
    assert p.info["path"] == path
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=15)
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * eps


@pytest.mark.parametrize("prec,path", SMALL_D_PATHS)
def test_small_d_wide_score_range(fs, prec, path):
    # The 250k-point 3-D recipe (unit cube against a tight 8-component
    # mixture, eps 0.01) at a small size: scores of one row span hundreds of
    # base-2 units, so the running maximum (the small-d matrix path's lazily
    # moved reference) changes many times, within and across tiles.
    w = workloads.make("c5", n=3000, m=2600)
    p, f, g, _, _ = gpu_solve(w.X, w.Y, w.a, w.b, eps=w.eps, iters=4, prec=prec)
    assert p.info["path"] == path
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=w.eps, iters=4)
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * w.eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * w.eps


@pytest.mark.parametrize("d", [1, 2, 3, 4])
def test_small_d_three_part_format(fs, d):
    # A small eps on unit-variance clouds: the fp16 split's bound (c_score
    # times the largest row sum of |x| times the largest |y|, under 2^9 on
    # centred points) fails for any centring, so d <= 4 takes the bf16
    # three-part records (six products per coordinate, two bf16 matrix
    # instructions per block) and must still meet the fp32 bar.  (The
    # products they drop are 2^-24 of c_score |x| |y|, as is the rounding of
    # the fp32 accumulation itself, so the bar holds while that product stays
    # within a few thousand base-2 units; it is about 2 * 10^3 here.)
    X, Y, a, b = _problem(900 + d, 1300, 1100, d, scale=1.0 / np.sqrt(d))
    eps = 0.015
    c_score = 2.0 / (eps * np.log(2.0))
    for o in (X.mean(0), Y.mean(0), 0.5 * (np.r_[X, Y].min(0) + np.r_[X, Y].max(0))):
        bound = c_score * np.abs(X - o).sum(1).max() * np.abs(Y - o).max()
        assert bound > 2 * 512, bound
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=6)
    assert p.info["path"] == "fp32-small-mfma"
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=6)
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * eps


@pytest.mark.parametrize("prec,path", SMALL_D_PATHS)
def test_small_d_splits(fs, prec, path):
    # Few rows, many keys: the key range is split across workgroups.
    X, Y, a, b = _problem(150, 1500, 24_000, 3, scale=0.5)
    eps = 0.02
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=3, prec=prec)
    assert p.info["path"] == path and p.info["f_splits"] > 1, p.info
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=3)
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * eps


@pytest.mark.parametrize("prec,path", SMALL_D_PATHS)
@pytest.mark.parametrize("n,m", [(1, 1), (3, 4), (40, 5), (9, 7), (600, 2), (2, 600)])
def test_small_d_tiny_sides(fs, prec, path, n, m):
    # Fewer keys than a lane half covers per block (m <= 4 leaves half of
    # every row's lanes without a key), and single points.
    X, Y, a, b = _problem(160 + n + m, n, m, 3)
    eps = 0.1
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=5, prec=prec)
    assert p.info["path"] == path
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=5)
    assert np.all(np.isfinite(host(f))) and np.all(np.isfinite(host(g)))
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * eps


@pytest.mark.parametrize("d,n,m", [(9, 700, 1100), (16, 1500, 900), (64, 2100, 1700),
                                   (100, 600, 1300), (256, 640, 500), (400, 900, 1300)])
def test_fp32_mfma_path(fs, d, n, m):
    X, Y, a, b = _problem(200 + d, n, m, d, scale=1.0 / np.sqrt(d))
    eps = 0.05
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=12)
    assert p.info["path"] == "fp32-mfma"
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=12)
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * eps


@pytest.mark.parametrize("prec", ["bf16", "fp16"])
@pytest.mark.parametrize("d,n,m", [(16, 900, 1300), (64, 1200, 1000), (200, 700, 650),
                                   (512, 1000, 900), (1024, 500, 700)])
def test_lowp_mfma_path(fs, prec, d, n, m):
    # The 50k x 50k, 512-D recipe's distribution (two 10-component Gaussian
    # mixtures, Dirichlet weights, eps 0.1) at small sizes and several d.
    w = workloads.make("c3", n=n, m=m, d=d)
    X, Y, a, b, eps = w.X, w.Y, w.a, w.b, w.eps
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=10, prec=prec)
    assert p.info["path"] == f"{prec}-mfma"
    rr = RoundedProblem(X, Y, prec).solve(a, b, eps=eps, iters=10)
    assert max_err(host(f), rr["f"]) <= TOL_LOWP_ROUNDED * eps
    assert max_err(host(g), rr["g"]) <= TOL_LOWP_ROUNDED * eps
    if prec == "bf16" and d < 64:
        # the original points' bar at this d: test_bf16_low_d_against_oracle
        return
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=10)
    assert max_err(host(f), ref["f"]) <= TOL_LOWP * eps
    assert max_err(host(g), ref["g"]) <= TOL_LOWP * eps


@pytest.mark.xfail(strict=True, reason=(
    "bf16 keeps 8 significant bits: at d = 16 on the two-mixture recipe the rounding of "
    "the centred points alone moves f by about 3e-2 eps, over the 2e-2 eps bar; the "
    "header documents bf16 as meeting the bar from d >= 64 on this recipe (fp16 and fp32 "
    "meet it at every d, test_lowp_mfma_path and test_fp32_mfma_path)"))
def test_bf16_low_d_against_oracle(fs):
    w = workloads.make("c3", n=900, m=1300, d=16)
    _, f, g, _, _ = gpu_solve(w.X, w.Y, w.a, w.b, eps=w.eps, iters=10, prec="bf16")
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=w.eps, iters=10)
    assert max_err(host(f), ref["f"]) <= TOL_LOWP * w.eps
    assert max_err(host(g), ref["g"]) <= TOL_LOWP * w.eps


@pytest.mark.parametrize("prec,d", [("fp16", 1024), ("bf16", 512), ("auto", 64)])
@pytest.mark.parametrize("n,m", [(1, 1), (1, 70), (70, 1), (33, 17)])
def test_matrix_paths_tiny_sides(fs, prec, d, n, m):
    # Single points and sides shorter than one tile on the matrix-core
    # kernels (the 1024-wide ones included): the solve and the transport.
    import torch
    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make("c4", n=n, m=m, d=d)
    eps = 0.05
    dv = 40
    p, f, g, _, _ = gpu_solve(w.X, w.Y, w.a, w.b, eps=eps, iters=4, prec=prec, dv_max=dv)
    V = np.random.default_rng(n + m).standard_normal((m, dv)).astype(np.float32)
    U = torch.empty((n, dv), device="cuda")
    binding.fs_apply_transport(p, eps, f, g, dev(V), U)
    torch.cuda.synchronize()
    fh, gh = host(f), host(g)
    assert np.all(np.isfinite(fh)) and np.all(np.isfinite(gh))
    if prec in ("bf16", "fp16"):
        rp = RoundedProblem(w.X, w.Y, prec)
        ref = rp.solve(w.a, w.b, eps=eps, iters=4)
        U_ref = rp.transport(w.a, w.b, fh, gh, V, eps)
        tol = TOL_LOWP_ROUNDED
    else:
        ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=eps, iters=4)
        U_ref = oracle.transport(w.X, w.Y, w.a, w.b, fh, gh, V, eps)
        tol = TOL_FP32
    assert max_err(fh, ref["f"]) <= tol * eps and max_err(gh, ref["g"]) <= tol * eps
    assert np.linalg.norm(host(U) - U_ref) <= 1e-3 * np.linalg.norm(U_ref)


def test_split_path_is_exercised(fs):
    # Sizes for which the launch heuristic splits the key range.
    X, Y, a, b = _problem(400, 4000, 3000, 64, scale=0.125)
    eps = 0.05
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=5)
    info = p.info
    assert info["f_splits"] > 1 and info["g_splits"] > 1, info
    ref = oracle_solve(X, Y, a, b, eps=eps, iters=5)
    assert max_err(host(f), ref["f"]) <= TOL_FP32 * eps
    assert max_err(host(g), ref["g"]) <= TOL_FP32 * eps


@pytest.mark.parametrize("prec", ["fp16", "bf16"])
def test_wide_rows_unsplit_with_residual(fs, prec):
    # 1024-D two-byte rows: 32,700 rows fill 256 row blocks of 128, so the
    # f-update runs unsplit (finalize and per-block residual in the kernel);
    # the g-update over those 32,700 keys runs split.  1,100 keys leave a
    # ragged last tile.  Sampled rows and columns against the oracle on the
    # path's own problem; the residual against its definition evaluated on
    # the GPU's own outputs.
    import torch
    from streaming_sinkhorn_solver_amd import binding

    n, m = 32700, 1100
    w = workloads.make("c4", n=n, m=m)
    eps = 0.05
    Xd, Yd, ad, bd = dev(w.X), dev(w.Y), dev(w.a), dev(w.b)
    f = torch.empty(n, device="cuda")
    g = torch.empty(m, device="cuda")
    p = binding.fs_potentials_init(Xd, Yd, ad, bd, prec=prec, f=f, g=g)
    assert p.info["f_splits"] == 1 and p.info["g_splits"] > 1, p.info
    binding.fs_sinkhorn_solve(p, f, g, eps_end=eps, iters_per_stage=3)
    f1 = torch.empty_like(f)
    g1 = torch.empty_like(g)
    r = torch.zeros(1, device="cuda")
    binding.fs_lse_update_f(p, eps, g, f1, f_cur=f, row_resid=r)
    binding.fs_lse_update_g(p, eps, f1, g1)
    torch.cuda.synchronize()
    fh, gh, f1h, g1h = host(f), host(g), host(f1), host(g1)
    rng = np.random.default_rng(77)
    rows = np.sort(np.concatenate([rng.choice(n, 200, replace=False), [0, 127, 128, n - 1]]))
    cols = np.sort(np.concatenate([rng.choice(m, 100, replace=False), [0, m - 1]]))
    rp = RoundedProblem(w.X, w.Y, prec)
    assert max_err(f1h[rows], rp.f_update_rows(w.b, gh, eps, rows)) <= TOL_LOWP_ROUNDED * eps
    assert max_err(g1h[cols], rp.g_update_cols(w.a, f1h, eps, cols)) <= TOL_LOWP_ROUNDED * eps
    want = float(np.sum(np.asarray(w.a, np.float64) *
                        np.abs(np.exp((fh.astype(np.float64) - f1h) / eps) - 1.0)))
    got = float(r.cpu()[0])
    assert abs(got - want) <= 1e-4 * want + 1e-7, (got, want)


def test_residual_matches_oracle(fs):
    import torch
    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b = _problem(500, 900, 1100, 3)
    eps = 0.3
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=7)
    out2 = torch.zeros(2, dtype=torch.float32, device="cuda")
    binding.fs_marginal_residual(p, eps, f, g, out2)
    torch.cuda.synchronize()
    tot, rt, ct = oracle.marginal_residual(X, Y, a, b, host(f), host(g), eps)
    r = out2.cpu().numpy()
    assert abs(r[0] - rt) <= 1e-3 * max(rt, 1e-6) + 1e-6
    assert abs(r[1] - ct) <= 1e-5


@pytest.mark.parametrize("prec,d,exact", [("fp32-valu", 3, True), ("auto", 32, True),
                                          ("bf16", 64, True), ("auto", 3, False)])
def test_power_of_two_scaling(fs, prec, d, exact):
    # Scaling the points by 2 and eps by 4 scales the potentials by 4.  Paths
    # whose arithmetic only sees power-of-two rescaled values reproduce it
    # bit for bit.  The small-d matrix path splits values into fp16 parts,
    # whose low parts can be subnormal (a fixed absolute grid that does not
    # rescale), so there the check is to within a tiny fraction of eps.
    X, Y, a, b = _problem(600 + d, 800, 700, d)
    eps = 0.25
    p1, f1, g1, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=6, prec=prec)
    _, f2, g2, _, _ = gpu_solve(2 * X, 2 * Y, a, b, eps=4 * eps, iters=6, prec=prec)
    if exact:
        np.testing.assert_array_equal(host(f2), 4 * host(f1))
        np.testing.assert_array_equal(host(g2), 4 * host(g1))
    else:
        assert p1.info["path"] == "fp32-small-mfma"
        assert max_err(host(f2), 4 * host(f1)) <= 1e-5 * 4 * eps
        assert max_err(host(g2), 4 * host(g1)) <= 1e-5 * 4 * eps


@pytest.mark.parametrize("prec,tol", [("fp32-valu", 1e-5), ("auto", 1e-4)])
def test_row_permutation(fs, prec, tol):
    # Permuting the points of X permutes f and leaves g unchanged, up to
    # rounding.  In the vector path only the order of the g-update's key sums
    # changes.  The small-d matrix path also folds each row's running
    # reference (taken from the keys that share the row's first block, so
    # dependent on the key order) into the score accumulation, which rounds
    # at the scale of the biased scores (about 2^-17 relative to |beta| of a
    # few hundred base-2 units here): an order-dependent difference of some
    # 1e-5 eps that five iterations carry along.
    X, Y, a, b = _problem(700, 1200, 900, 3)
    perm = np.random.default_rng(701).permutation(1200)
    eps = 0.2
    _, f1, g1, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=5, prec=prec)
    _, f2, g2, _, _ = gpu_solve(X[perm], Y, a[perm], b, eps=eps, iters=5, prec=prec)
    assert max_err(host(f2), host(f1)[perm]) <= tol * eps
    assert max_err(host(g2), host(g1)) <= tol * eps


def test_deterministic_repeat(fs):
    X, Y, a, b = _problem(800, 3000, 2500, 64, scale=0.125)
    _, f1, g1, _, _ = gpu_solve(X, Y, a, b, eps=0.05, iters=4)
    _, f2, g2, _, _ = gpu_solve(X, Y, a, b, eps=0.05, iters=4)
    np.testing.assert_array_equal(host(f1), host(f2))
    np.testing.assert_array_equal(host(g1), host(g2))


# (precision, d, width of V): the vector paths (d = 3), the streaming matrix
# kernel with 128-column blocks (dv <= 128) and 256-column blocks (two
# blocks for dv = 300, one ragged), key-range splits with their merge (the
# launch heuristic splits these small row counts), and the 1024-D kernel.
@pytest.mark.parametrize("prec,d,dv", [("auto", 3, 70), ("fp32-valu", 3, 70), ("auto", 64, 70),
                                       ("auto", 64, 300), ("bf16", 512, 70),
                                       ("bf16", 512, 300), ("fp16", 256, 70),
                                       ("fp16", 128, 513), ("fp16", 1024, 100)])
def test_transport(fs, prec, d, dv):
    import torch
    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b = _problem(900 + d, 700, 850, d, scale=1.0 / np.sqrt(d))
    rng = np.random.default_rng(901 + dv)
    V = rng.standard_normal((850, dv)).astype(np.float32)
    eps = 0.1
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=8, prec=prec, dv_max=max(dv, 128))
    Vd = dev(V)
    U = torch.empty((700, dv), dtype=torch.float32, device="cuda")
    T = torch.empty((700, dv), dtype=torch.float32, device="cuda")
    binding.fs_apply_transport(p, eps, f, g, Vd, U, divide_by_a=False)
    binding.fs_apply_transport(p, eps, f, g, Vd, T, divide_by_a=True)
    torch.cuda.synchronize()
    if prec in ("bf16", "fp16"):
        rp = RoundedProblem(X, Y, prec)
        U_ref = rp.transport(a, b, host(f), host(g), V, eps)
        T_ref = rp.transport(a, b, host(f), host(g), V, eps, divide_by_a=True)
    else:
        U_ref = oracle.transport(X, Y, a, b, host(f), host(g), V, eps)
        T_ref = oracle.transport(X, Y, a, b, host(f), host(g), V, eps, divide_by_a=True)
    for got, ref in ((host(U), U_ref), (host(T), T_ref)):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 1e-3, rel


# The streaming kernels take their row references from the row potential:
# with potentials far from consistent (some rows' f raised by 1, weights near
# 2^24 against that reference; others lowered by 3, weights near 2^-33) the
# marked rows' blocks are recomputed against their score maxima.  Rows left
# alone keep their first-pass result, so both kinds of block occur; one and
# several key ranges, one and two 512-column blocks, and the 1024-wide
# kernel (64-row blocks).
@pytest.mark.parametrize("prec,d,dv,m", [("auto", 64, 300, 850), ("bf16", 512, 300, 850),
                                         ("fp16", 256, 513, 850), ("bf16", 512, 512, 20000),
                                         ("fp16", 1024, 300, 850), ("bf16", 1024, 1024, 3000)])
def test_transport_inconsistent_potentials(fs, prec, d, dv, m):
    import torch
    from streaming_sinkhorn_solver_amd import binding

    n = 700
    X, Y, a, b = _problem(1900 + d, n, m, d, scale=1.0 / np.sqrt(d))
    V = np.random.default_rng(1901 + dv).standard_normal((m, dv)).astype(np.float32)
    eps = 0.1
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=8, prec=prec, dv_max=dv)
    fh = host(f).astype(np.float32)
    shift = np.zeros(n, np.float32)
    shift[0:n:3] = 1.0
    shift[1:n:7] = -3.0
    shift[256:384] = 0.0  # a 128-row block (two 64-row blocks) without a marked row
    fs_ = (fh + shift).astype(np.float32)
    U = torch.empty((n, dv), dtype=torch.float32, device="cuda")
    T = torch.empty((n, dv), dtype=torch.float32, device="cuda")
    binding.fs_apply_transport(p, eps, dev(fs_), g, dev(V), U)
    binding.fs_apply_transport(p, eps, dev(fs_), g, dev(V), T, divide_by_a=True)
    torch.cuda.synchronize()
    if prec in ("bf16", "fp16"):
        rp = RoundedProblem(X, Y, prec)
        U_ref = rp.transport(a, b, fs_, host(g), V, eps)
        T_ref = rp.transport(a, b, fs_, host(g), V, eps, divide_by_a=True)
    else:
        U_ref = oracle.transport(X, Y, a, b, fs_, host(g), V, eps)
        T_ref = oracle.transport(X, Y, a, b, fs_, host(g), V, eps, divide_by_a=True)
    for got, ref in ((host(U), U_ref), (host(T), T_ref)):
        assert np.all(np.isfinite(got))
        # row by row: the shifted rows' scales differ by e^40
        num = np.linalg.norm(got - ref, axis=1)
        den = np.linalg.norm(ref, axis=1)
        assert np.max(num / den) <= 1e-3, np.max(num / den)


# The d <= 8 transport: every column-block width (dv = 1, 2, 4, 5, 16 and
# 33, i.e. 1 to 32 columns per thread and two blocks), one and several rows
# per thread (the larger row count fills enough workgroups for the latter),
# and a key count that leaves a ragged tile of the LDS-staged key loop.
@pytest.mark.parametrize("prec,d,dv,n", [("auto", 3, 1, 700), ("fp32-valu", 8, 2, 700),
                                         ("auto", 5, 4, 1100), ("auto", 3, 5, 1_050_000),
                                         ("fp32-valu", 3, 16, 700), ("auto", 7, 33, 700)])
def test_transport_small_d(fs, prec, d, dv, n):
    import torch
    from streaming_sinkhorn_solver_amd import binding

    m = 850
    X, Y, a, b = _problem(950 + d + dv, n, m, d, scale=1.0 / np.sqrt(d))
    V = np.random.default_rng(dv).standard_normal((m, dv)).astype(np.float32)
    eps = 0.1
    p, f, g, _, _ = gpu_solve(X, Y, a, b, eps=eps, iters=4, prec=prec, dv_max=dv)
    U = torch.empty((n, dv), dtype=torch.float32, device="cuda")
    binding.fs_apply_transport(p, eps, f, g, dev(V), U)
    torch.cuda.synchronize()
    rows = None if n <= 2000 else np.sort(np.concatenate(
        [np.random.default_rng(1).choice(n, 200, replace=False), [0, 1023, 1024, n - 1]]))
    ref = oracle.transport(X, Y, a, b, host(f), host(g), V, eps, rows=rows)
    got = host(U) if rows is None else host(U)[rows]
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 1e-3, rel


# The 1024-D streaming transport: every output-block width (dv = 40, 100,
# 200, 300 and 1024 use 1, 2, 4, 8 and 16 blocks of 32 columns per wave),
# two column blocks (dv = 1100), key counts that leave a ragged 16-key tile,
# and the key-range splits the launch heuristic picks for these few rows
# (and none at 6,000 rows).
@pytest.mark.parametrize("prec,dv,n,m", [("fp16", 40, 700, 850), ("bf16", 100, 500, 1000),
                                         ("fp16", 200, 300, 777), ("fp16", 300, 700, 850),
                                         ("bf16", 1024, 400, 601), ("fp16", 1100, 260, 500),
                                         ("fp16", 1024, 6000, 333)])
def test_transport_wide_rows(fs, prec, dv, n, m):
    import torch
    from streaming_sinkhorn_solver_amd import binding

    w = workloads.make("c4", n=n, m=m)
    rng = np.random.default_rng(dv + n)
    V = rng.standard_normal((m, dv)).astype(np.float32)
    eps = 0.05
    p, f, g, _, _ = gpu_solve(w.X, w.Y, w.a, w.b, eps=eps, iters=5, prec=prec, dv_max=dv)
    U = torch.empty((n, dv), dtype=torch.float32, device="cuda")
    T = torch.empty((n, dv), dtype=torch.float32, device="cuda")
    Vd = dev(V)
    binding.fs_apply_transport(p, eps, f, g, Vd, U)
    binding.fs_apply_transport(p, eps, f, g, Vd, T, divide_by_a=True)
    torch.cuda.synchronize()
    rows = None if n <= 1000 else np.sort(np.concatenate(
        [rng.choice(n, 120, replace=False), [0, 63, 64, n - 1]]))
    rp = RoundedProblem(w.X, w.Y, prec)
    U_ref = rp.transport(w.a, w.b, host(f), host(g), V, eps, rows=rows)
    T_ref = rp.transport(w.a, w.b, host(f), host(g), V, eps, divide_by_a=True, rows=rows)
    for got, ref in ((host(U), U_ref), (host(T), T_ref)):
        got = got if rows is None else got[rows]
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 1e-3, rel


def _c4_annealed(prec):
    # The annealed 1024-D recipe (eps 1 -> 0.01) at a small size.
    w = workloads.make("c4", n=600, m=500)
    _, f, g, info, _ = gpu_solve(w.X, w.Y, w.a, w.b, eps=w.eps, eps_start=w.eps_start,
                                 n_stages=4, iters=6, prec=prec)
    assert info["iters_done"] == 24
    return w, f, g


def test_annealing_matches_rounded_oracle(fs):
    # Kernel exactness on the annealed schedule: the fp16 path solves the
    # problem of the rounded centred clouds exactly up to fp32.
    w, f, g = _c4_annealed("fp16")
    rr = RoundedProblem(w.X, w.Y, "fp16").solve(w.a, w.b, eps=w.eps, eps_start=w.eps_start,
                                                n_stages=4, iters=6)
    assert max_err(host(f), rr["f"]) <= TOL_LOWP_ROUNDED * w.eps
    assert max_err(host(g), rr["g"]) <= TOL_LOWP_ROUNDED * w.eps


def test_annealing_fp16_against_oracle(fs):
    # The parity bar on the original points at the final eps = 0.01: fp16
    # rounding of the centred 1024-D points moves f by about 5e-3 eps here.
    w, f, g = _c4_annealed("fp16")
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=w.eps, eps_start=w.eps_start, n_stages=4, iters=6)
    assert max_err(host(f), ref["f"]) <= TOL_LOWP * w.eps
    assert max_err(host(g), ref["g"]) <= TOL_LOWP * w.eps


@pytest.mark.xfail(strict=True, reason=(
    "bf16 keeps 8 significant bits: on the annealed 1024-D recipe at eps = 0.01 "
    "the rounding of the centred points alone moves f by about 4.5e-2 eps, over "
    "the 2e-2 eps bar; that recipe runs in fp16 (same matrix-core rate)"))
def test_annealing_bf16_against_oracle(fs):
    w, f, g = _c4_annealed("bf16")
    ref = oracle_solve(w.X, w.Y, w.a, w.b, eps=w.eps, eps_start=w.eps_start, n_stages=4, iters=6)
    assert max_err(host(f), ref["f"]) <= TOL_LOWP * w.eps
    assert max_err(host(g), ref["g"]) <= TOL_LOWP * w.eps


def test_tol_stop(fs):
    X, Y, a, b = _problem(1000, 500, 400, 3)
    _, f, g, info, _ = gpu_solve(X, Y, a, b, eps=0.5, iters=2000, tol=1e-4, check_every=5)
    assert info["status"] == 0 and 0 < info["iters_done"] < 2000
    assert info["iters_done"] % 5 == 0
    tot, _, _ = oracle.marginal_residual(X, Y, a, b, host(f), host(g), 0.5)
    assert tot <= 2e-4
    # unreachable tolerance: NOT_CONVERGED with valid outputs
    _, f, g, info, _ = gpu_solve(X, Y, a, b, eps=0.5, iters=3, tol=1e-12, check_every=2)
    assert info["status"] == 5 and info["iters_done"] == 3
    assert np.all(np.isfinite(host(f)))


def test_error_paths(fs):
    import torch
    from streaming_sinkhorn_solver_amd import binding

    X, Y, a, b = _problem(1100, 64, 48, 3)
    Xb = X.copy()
    Xb[5, 1] = np.nan
    with pytest.raises(binding.FsError) as e:
        binding.fs_potentials_init(dev(Xb), dev(Y), dev(a), dev(b))
    assert e.value.status == binding.FS_ERR_NONFINITE
    a0 = a.copy()
    a0[3] = 0.0
    with pytest.raises(binding.FsError) as e:
        binding.fs_potentials_init(dev(X), dev(Y), dev(a0), dev(b))
    assert e.value.status == binding.FS_ERR_NONFINITE
    small = torch.empty(128, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.FsError) as e:
        binding.fs_potentials_init(dev(X), dev(Y), dev(a), dev(b), workspace=small)
    assert e.value.status == binding.FS_ERR_WORKSPACE
    p = binding.fs_potentials_init(dev(X), dev(Y), dev(a), dev(b))
    f = torch.zeros(64, device="cuda")
    g = torch.zeros(48, device="cuda")
    with pytest.raises(binding.FsError) as e:
        binding.fs_lse_update_f(p, -1.0, g, f)
    assert e.value.status == binding.FS_ERR_INVALID_ARG
    r = torch.zeros(1, device="cuda")
    with pytest.raises(binding.FsError) as e:
        binding.fs_lse_update_f(p, 0.1, g, f, f_cur=f, row_resid=r)
    assert e.value.status == binding.FS_ERR_INVALID_ARG
