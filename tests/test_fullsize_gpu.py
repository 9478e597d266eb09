"""Full-size spot checks: each recipe at its real shape, in the precision and
launch configuration bench.py times (same sizes, same score path, hence the
same key-range splits and workgroup counts).

After a few GPU iterations at the recipe's final eps, one more GPU f-update
and g-update are compared, on 512 seeded rows and columns, with the oracle's
single update from the same GPU potentials.  This isolates one update's
error from trajectory drift at a cost of 512 m d + 512 n d per check.  Two
references:

  * the oracle on the original points, at the parity bar (max over the
    sampled entries): 1e-3 eps for fp32 score paths, 2e-2 eps for bf16/fp16;
  * the oracle on the problem the path actually solves (each cloud centred on
    its own bounding-box midpoint, the centred points rounded to the score
    type, fp32 per-point cost terms), at a bar from the arithmetic of each
    path that a kernel mistake would exceed:
      fp32 matrix path (C2, d = 64)   1e-4  fp32 rounding of the expanded
                                            score c_score x.y + beta (|z2| ~
                                            1e2 in base-2 units): ~1e-5 eps
      bf16 path (C3)                  1e-4  fp32 accumulation of 512 exact
                                            products: ~sqrt(d) 2^-24 c_score
                                            |x.y| ~ 3e-5 eps at eps = 0.1
      fp16 path (C4)                  5e-4  the same at d = 1024, eps = 0.01:
                                            ~1e-4 to 4e-4 eps (little
                                            averaging over keys in a
                                            concentrated plan)
      d = 3 matrix path (C1, C5)      2e-4  the fp16 split's ~2^-21 relative
                                            error per product under the path's
                                            guard (c_score * max L1 * max|y|
                                            <= 2^9)
"""
import numpy as np
import pytest

import oracle
from helpers import RoundedProblem, dev, host
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu

# recipe -> (score precision, tolerance against the path's own problem in
# eps, expected path)
RECIPES = {
    "c1": ("auto", 2e-4, "fp32-small-mfma"),
    "c2": ("fp32", 1e-4, "fp32-mfma"),
    "c3": ("bf16", 1e-4, "bf16-mfma"),
    "c4": ("fp16", 5e-4, "fp16-mfma"),
    "c5": ("auto", 2e-4, "fp32-small-mfma"),
}
SAMPLES = 512
WARM_ITERS = 3


@pytest.mark.parametrize("name", sorted(RECIPES))
def test_full_size_one_step(fs, name):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    prec, tol, path = RECIPES[name]
    w = workloads.make(name)
    Xd, Yd, ad, bd = dev(w.X), dev(w.Y), dev(w.a), dev(w.b)
    f = torch.empty(w.n, device="cuda")
    g = torch.empty(w.m, device="cuda")
    p = binding.fs_potentials_init(Xd, Yd, ad, bd, prec=prec, f=f, g=g)
    assert p.info["path"] == path
    binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=WARM_ITERS)
    f1 = torch.empty_like(f)
    g1 = torch.empty_like(g)
    binding.fs_lse_update_f(p, w.eps, g, f1)
    binding.fs_lse_update_g(p, w.eps, f1, g1)
    torch.cuda.synchronize()
    gh, f1h, g1h = host(g), host(f1), host(g1)
    assert np.all(np.isfinite(f1h)) and np.all(np.isfinite(g1h))

    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(w.n, size=min(SAMPLES, w.n), replace=False))
    cols = np.sort(rng.choice(w.m, size=min(SAMPLES, w.m), replace=False))
    rp = RoundedProblem(w.X, w.Y, prec if prec in ("bf16", "fp16") else "fp32")
    ef = float(np.max(np.abs(f1h[rows] - rp.f_update_rows(w.b, gh, w.eps, rows)))) / w.eps
    eg = float(np.max(np.abs(g1h[cols] - rp.g_update_cols(w.a, f1h, w.eps, cols)))) / w.eps
    uf = float(np.max(np.abs(f1h[rows] - oracle.f_update_rows(w.X, w.Y, w.b, gh, w.eps, rows))))
    ug = float(np.max(np.abs(g1h[cols] - oracle.g_update_cols(w.X, w.Y, w.a, f1h, w.eps, cols))))
    bar = 2e-2 if prec in ("bf16", "fp16") else 1e-3
    print(f"{name}: path's problem f {ef:.2e} g {eg:.2e} eps (tolerance {tol:g}); original "
          f"points f {uf / w.eps:.2e} g {ug / w.eps:.2e} eps (bar {bar:g}); splits "
          f"{p.info['f_splits']}/{p.info['g_splits']}")
    assert ef <= tol and eg <= tol
    assert uf <= bar * w.eps and ug <= bar * w.eps


# recipe -> rows sampled for the transport check
TRANSPORT = {"c3": 64, "c4": 32}


@pytest.mark.parametrize("name", sorted(TRANSPORT))
def test_full_size_transport(fs, name):
    """The transport at full size, in the launch configuration bench.py times
    (same shapes, so the same column blocks and key-range splits), on sampled
    rows against the oracle on the path's own problem; parity bar 1e-3
    relative (Frobenius over the sampled rows)."""
    import torch

    from streaming_sinkhorn_solver_amd import binding

    prec, _, path = RECIPES[name]
    w = workloads.make(name)
    Xd, Yd, ad, bd, Vd = dev(w.X), dev(w.Y), dev(w.a), dev(w.b), dev(w.V)
    dv = w.V.shape[1]
    f = torch.empty(w.n, device="cuda")
    g = torch.empty(w.m, device="cuda")
    p = binding.fs_potentials_init(Xd, Yd, ad, bd, prec=prec, f=f, g=g, dv_max=dv)
    assert p.info["path"] == path
    binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=WARM_ITERS)
    U = torch.empty((w.n, dv), device="cuda")
    binding.fs_apply_transport(p, w.eps, f, g, Vd, U, divide_by_a=w.divide_by_a)
    torch.cuda.synchronize()
    Uh = host(U)
    assert np.all(np.isfinite(Uh))
    rows = np.sort(np.random.default_rng(77).choice(w.n, size=TRANSPORT[name], replace=False))
    rp = RoundedProblem(w.X, w.Y, prec)
    ref = rp.transport(w.a, w.b, host(f), host(g), w.V, w.eps, divide_by_a=w.divide_by_a,
                       rows=rows)
    rel = np.linalg.norm(Uh[rows] - ref) / np.linalg.norm(ref)
    worst = np.max(np.linalg.norm(Uh[rows] - ref, axis=1) / np.linalg.norm(ref, axis=1))
    print(f"{name} transport: relative error {rel:.2e} (worst row {worst:.2e}) on "
          f"{len(rows)} rows")
    assert rel <= 1e-3


def test_full_size_hvp_symmetry(fs):
    """The Hessian-vector product at the 50k x 50k x 512 recipe's full size
    (bf16, the one-pass second moment, the launch heuristic's key-range
    splits), where the dense oracle cannot go: <U, H V> = <V, H U> for two
    seeded directions, and H V finite.  Bar 5e-3 relative, the bf16 HVP bar
    (tests/test_hvp_gpu.py)."""
    import torch

    from streaming_sinkhorn_solver_amd import binding

    prec = RECIPES["c3"][0]
    w = workloads.make("c3")
    Xd, Yd, ad, bd = dev(w.X), dev(w.Y), dev(w.a), dev(w.b)
    f = torch.empty(w.n, device="cuda")
    g = torch.empty(w.m, device="cuda")
    p = binding.fs_potentials_init(Xd, Yd, ad, bd, prec=prec, f=f, g=g, dv_max=w.d + 2)
    binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=20)
    rng = np.random.default_rng(5)
    U, V = (rng.standard_normal((w.n, w.d)).astype(np.float32) for _ in range(2))
    HU, HV = torch.empty((w.n, w.d), device="cuda"), torch.empty((w.n, w.d), device="cuda")
    scratch = torch.empty(binding.fs_hvp_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    iu = binding.fs_hvp(p, w.eps, f, g, Xd, Yd, dev(U), HU, workspace=scratch)
    iv = binding.fs_hvp(p, w.eps, f, g, Xd, Yd, dev(V), HV, workspace=scratch)
    torch.cuda.synchronize()
    hu, hv = host(HU), host(HV)
    assert np.all(np.isfinite(hu)) and np.all(np.isfinite(hv))
    lhs = float(np.sum(U.astype(np.float64) * hv))
    rhs = float(np.sum(V.astype(np.float64) * hu))
    print(f"c3 HVP symmetry: {lhs:.6e} vs {rhs:.6e}; CG {iu} {iv}")
    assert abs(lhs - rhs) <= 5e-3 * max(abs(lhs), abs(rhs))


# (recipe, eps override, delta): the c5 clouds at their own eps and in the
# blur-equals-spacing regime, and the uniform pair of the block-sparse form
BLOCK_SPARSE = [("c5", None, 1e-3), ("c5", 250_000 ** (-2 / 3), 1e-3), ("fs2", None, 1e-3)]


@pytest.mark.parametrize("name,eps,delta", BLOCK_SPARSE)
def test_full_size_block_sparse(fs, name, eps, delta):
    """The block-sparse form at 250k x 250k (d = 3) in the configuration
    bench.py times (GPU Morton order, annealed block-sparse solve to the
    final eps), then one more f- and g-update compared on 512 sampled rows
    and columns with the dense oracle update through the certificate
    (-tol <= new - dense <= eps log(1 + delta exp((new - cur)/eps)) + tol,
    tol = 1e-3 eps), and two row blocks' skipped key blocks checked by
    brute force against the mass bound."""
    import torch

    from oracle import blocksparse as obs

    B = fs
    w = workloads.make(name)
    eps = w.eps if eps is None else eps
    Xs, a_s, px = B.fs_morton_sort(dev(w.X), dev(w.a))
    Ys, b_s, py = B.fs_morton_sort(dev(w.Y), dev(w.b))
    torch.cuda.synchronize()
    assert np.array_equal(px.cpu().numpy(), obs.morton_order(w.X))
    X, Y, a, b = host(Xs), host(Ys), host(a_s), host(b_s)
    f = torch.zeros(w.n, device="cuda")
    g = torch.zeros(w.m, device="cuda")
    p = B.fs_potentials_init(Xs, Ys, a_s, b_s, f=f, g=g)
    B.fs_bs_attach(p)
    B.fs_bs_sinkhorn_solve(p, f, g, eps_end=eps, eps_start=0.1, n_stages=12,
                           iters_per_stage=10, delta=delta)
    f_new = torch.empty_like(f)
    B.fs_bs_lse_update_f(p, eps, delta, g, f, f_new)
    torch.cuda.synchronize()
    fc, gc, fn = host(f), host(g), host(f_new)
    cnt_f, lists_f = B.fs_bs_read_screen(p, 0, lists=True)
    g_new = torch.empty_like(g)
    B.fs_bs_lse_update_g(p, eps, delta, f_new, g, g_new)
    torch.cuda.synchronize()
    gn = host(g_new)
    rng = np.random.default_rng(88)
    rows = np.sort(rng.choice(w.n, SAMPLES, replace=False))
    cols = np.sort(rng.choice(w.m, SAMPLES, replace=False))
    ref_f = oracle.f_update_rows(X, Y, b, gc, eps, rows)
    ref_g = oracle.g_update_cols(X, Y, a, fn, eps, cols)
    for new, ref, cur, idx in ((fn, ref_f, fc, rows), (gn, ref_g, gc, cols)):
        diff = new[idx] - ref
        cert = obs.certificate(new[idx], cur[idx], eps, delta)
        print(f"{name} eps {eps:.3g}: diff [{diff.min() / eps:.2e}, {diff.max() / eps:.2e}] eps, "
              f"certificate max {cert.max() / eps:.2e} eps")
        assert diff.min() >= -1e-3 * eps
        assert np.all(diff <= cert + 1e-3 * eps)
    # the barycentric projection over the kept blocks on the sampled rows:
    # |U - U_dense| <= delta max|Y| + 2e-3 (P.|Y| / a) (the skipped mass, fp32)
    Ub = torch.empty((w.n, 3), device="cuda")
    B.fs_bs_apply_transport(p, eps, delta, f_new, g_new, Ys, Ub, divide_by_a=True)
    torch.cuda.synchronize()
    ref_u = oracle.transport(X, Y, a, b, fn, gn, Y, eps, divide_by_a=True, rows=rows)
    ref_ua = oracle.transport(X, Y, a, b, fn, gn, np.abs(Y), eps, divide_by_a=True, rows=rows)
    du = np.abs(host(Ub)[rows] - ref_u)
    print(f"  barycentric projection: max error {du.max():.2e} (skip bound {delta * np.abs(Y).max():.2e})")
    assert np.all(du <= delta * np.abs(Y).max() + 2e-3 * ref_ua)
    # the gradient over the kept blocks on the sampled rows, by brute force in
    # float64: 2 sum_j P_ij (x_i - y_j), within 2 delta a_i max_j |x_ic - y_jc|
    # + 2e-3 (2 sum_j P_ij |x_ic - y_jc|) + 1e-5 a_i
    gx = torch.empty((w.n, 3), device="cuda")
    B.fs_bs_gradient(p, eps, delta, f_new, g_new, grad_x=gx)
    torch.cuda.synchronize()
    gxs = host(gx)[rows]
    Y64 = Y.astype(np.float64)
    worst = 0.0
    for r0 in range(0, len(rows), 16):
        rr = rows[r0:r0 + 16]
        D = X[rr].astype(np.float64)[:, None, :] - Y64[None, :, :]
        P = a[rr, None].astype(np.float64) * b[None, :] * np.exp(
            (fn[rr, None].astype(np.float64) + gn[None, :] - (D ** 2).sum(-1)) / eps)
        ref = 2 * np.einsum("ij,ijc->ic", P, D)
        absD = np.abs(D)
        env = (2 * delta * a[rr, None] * absD.max(axis=1)
               + 2e-3 * 2 * np.einsum("ij,ijc->ic", P, absD) + 1e-5 * a[rr, None])
        err = np.abs(gxs[r0:r0 + 16] - ref)
        worst = max(worst, float((err / env).max()))
        assert np.all(err <= env)
    print(f"  gradient: largest error / envelope {worst:.2e}")
    # brute-force mass of the skipped blocks of two row blocks (f side)
    nbK = (w.m + 31) // 32
    for I in (0, len(cnt_f) // 2):
        kept = lists_f[I, :cnt_f[I]]
        skip = np.setdiff1d(np.arange(nbK), kept)
        r = np.arange(I * 256, min(I * 256 + 256, w.n))
        keys = np.concatenate([np.arange(J * 32, min(J * 32 + 32, w.m)) for J in skip])
        blk = np.repeat(np.arange(len(skip)), [min(J * 32 + 32, w.m) - J * 32 for J in skip])
        mass = np.zeros((len(r), len(skip)))
        for c0 in range(0, len(keys), 65536):
            kk = keys[c0:c0 + 65536]
            C = ((X[r, None, :] - Y[None, kk, :]) ** 2).sum(-1)
            z = b[kk][None, :] * np.exp((fc[r, None] + gc[None, kk] - C) / eps)
            np.add.at(mass.T, blk[c0:c0 + 65536], z.T)
        print(f"  row block {I}: kept {len(kept)} of {nbK} key blocks, largest skipped mass "
              f"{mass.max():.2e} (bound {delta / nbK:.2e})")
        assert mass.max() < delta / nbK * 1.001


def test_full_size_coarse_stage_and_pipeline(fs):
    """The two-stage solve of the block-sparse form at 250k x 250k (the
    bench's fs2 pipeline): centroids against the oracle's (1e-6 relative),
    the sampled check against the oracle's on the lifted potentials (1e-4
    relative), then the block-sparse solve from the lift to a 1% residual,
    whose result is checked against the dense oracle update on 512 sampled
    rows through the certificate (the last g-update makes the columns exact,
    so the rows carry the residual)."""
    import torch

    from oracle import blocksparse as obs
    from oracle import coarse as oc

    B = fs
    w = workloads.make("fs2")
    eps, cell = w.eps, 8
    Xs, a_s, _ = B.fs_morton_sort(dev(w.X), dev(w.a))
    Ys, b_s, _ = B.fs_morton_sort(dev(w.Y), dev(w.b))
    X, Y, a, b = host(Xs), host(Ys), host(a_s), host(b_s)
    CX, WX = B.fs_centroids(Xs, a_s, cell)
    CY, WY = B.fs_centroids(Ys, b_s, cell)
    torch.cuda.synchronize()
    cx_ref, wx_ref = oc.centroids(X, a, cell)
    np.testing.assert_allclose(host(WX), wx_ref, rtol=1e-6)
    np.testing.assert_allclose(host(CX), cx_ref, rtol=1e-6, atol=1e-7)
    rng = np.random.default_rng(12)
    rows = rng.choice(w.n, 64, replace=False).astype(np.int32)
    cols = rng.choice(w.m, 64, replace=False).astype(np.int32)
    F = torch.empty(CX.shape[0], device="cuda")
    G = torch.empty(CY.shape[0], device="cuda")
    pc = B.fs_potentials_init(CX, CY, WX, WY, f=F, g=G)
    f = torch.empty(w.n, device="cuda")
    g = torch.empty(w.m, device="cuda")
    info = B.fs_bs_coarse_start(pc, Xs, Ys, a_s, b_s, cell, f, g, F, G,
                                torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda(),
                                eps_end=eps, eps_start=0.1, n_stages=12, iters_per_stage=10,
                                more_iters=20, check_tol=0.5, max_rounds=2)
    torch.cuda.synchronize()
    ref = oc.sampled_marginal_error(X, Y, a, b, host(f), host(g), eps, rows, cols)
    print(f"coarse stage: {info}; oracle check {ref}")
    np.testing.assert_allclose([info["err_rows"], info["err_cols"]], ref, rtol=1e-4)
    p = B.fs_potentials_init(Xs, Ys, a_s, b_s)
    B.fs_bs_attach(p)
    sol = B.fs_bs_sinkhorn_solve(p, f, g, eps_end=eps, iters_per_stage=3000, delta=1e-3,
                                 tol=1e-2, check_every=10, warm_start=True)
    assert sol["residual"] <= 1e-2
    f_cur = host(f).copy()
    f_new = torch.empty_like(f)
    B.fs_bs_lse_update_f(p, eps, 1e-3, g, f, f_new)
    torch.cuda.synchronize()
    sample = np.sort(rng.choice(w.n, SAMPLES, replace=False))
    ref_f = oracle.f_update_rows(X, Y, b, host(g), eps, sample)
    fn = host(f_new)[sample]
    diff = fn - ref_f
    cert = obs.certificate(fn, f_cur[sample], eps, 1e-3)
    print(f"pipeline: {sol['iters_done']} iterations, residual {sol['residual']:.2e}; "
          f"f diff [{diff.min() / eps:.2e}, {diff.max() / eps:.2e}] eps")
    assert diff.min() >= -1e-3 * eps
    assert np.all(diff <= cert + 1e-3 * eps)
