"""Pins of the block-sparse oracle (oracle/blocksparse.py).

The page gives no formula for the ordering, the screening threshold or the
error bound; the oracle's are a reading of it (see its header).  Pinned by
what that reading does not use:

B1  bit interleaving against a recursive Z-order enumeration of the grid
    (quadrants / octants visited in index order, each recursively);
B2  quantisation: the box corners map to cells 0 and 2^B - 1, cells are
    monotone in each coordinate, a flat axis maps to 0, ties keep index order;
B3  the box gap is a lower bound of every pair cost of two blocks (brute
    force) and exact for one-point blocks; the pair bounds H (the maximum of
    u.x + v.y - |x - y|^2 over two boxes) and H2 (of u.x + v.y + 2 x.y) are
    above their values at every pair of points and every point of a fine
    grid of the boxes, and attained on it;
B4  delta = 0 keeps every block: the update equals the dense oracle update;
B5  every skipped block's true mass (brute force over its pairs) is below
    delta / N_J of the row's target, so the skipped mass of a row is below
    delta * a_i;
    The two-level form (chunks of blocks skipped whole on a bound of their
    own) passes the same brute-force check;
B6  the certificate: 0 <= f_sparse - f_dense <= eps log(1 + delta
    exp((f_sparse - f_cur)/eps)) against the dense update, on problems where
    blocks are skipped;
B7  planted slips (a wrong sign in the edge maximiser, the mean residual of
    the row fit in place of its maximum) are caught by B3/B5.
"""
import numpy as np
import pytest

import oracle
from oracle import blocksparse as bs


def _z_order(k, d):
    """Cells of a 2^k-per-axis grid in recursive Z order."""
    if k == 0:
        return [(0,) * d]
    sub = _z_order(k - 1, d)
    half = 1 << (k - 1)
    out = []
    for o in range(1 << d):
        for cell in sub:
            out.append(tuple(((o >> c) & 1) * half + cell[c] for c in range(d)))
    return out


@pytest.mark.parametrize("d,k", [(1, 5), (2, 4), (3, 3)])
def test_b1_interleave_is_z_order(d, k):
    cells = _z_order(k, d)
    codes = bs.interleave(np.array(cells), d)
    assert np.array_equal(codes, np.arange(len(cells)))


def test_b2_quantise_endpoints_monotone_flat_and_ties():
    rng = np.random.default_rng(3)
    X = rng.uniform(-2.0, 5.0, (400, 3)).astype(np.float32)
    X[:, 2] = 1.25  # flat axis
    q = bs.quantize(X)
    B = bs.morton_bits(3)
    for c in range(2):
        assert q[np.argmin(X[:, c]), c] == 0
        assert q[np.argmax(X[:, c]), c] == (1 << B) - 1
        o = np.argsort(X[:, c], kind="stable")
        assert np.all(np.diff(q[o, c]) >= 0)
    assert np.all(q[:, 2] == 0)
    # duplicates keep their index order
    Xd = np.repeat(X[:5], 3, axis=0)
    perm = bs.morton_order(Xd)
    for r in range(5):
        pos = [int(np.nonzero(perm == 3 * r + t)[0][0]) for t in range(3)]
        assert pos == sorted(pos)


def test_b2_order_groups_cells():
    # points on a 4^3 grid of well-separated clusters: a cluster's points are
    # contiguous in the order and the clusters follow the Z-order of their cells
    rng = np.random.default_rng(4)
    cells = _z_order(2, 3)
    pts, lab = [], []
    for idx, c in enumerate(rng.permutation(len(cells))):
        centre = (np.array(cells[c]) + 0.5) / 4.0
        pts.append(centre + rng.uniform(-0.02, 0.02, (5, 3)))
        lab += [c] * 5
    X = np.concatenate(pts).astype(np.float32)
    X = np.concatenate([X, [[0, 0, 0], [1, 1, 1]]]).astype(np.float32)  # box = unit cube
    lab = np.array(lab + [-1, -2])
    seq = lab[bs.morton_order(X)]
    seq = seq[seq >= 0]
    runs = [seq[0]] + [v for p, v in zip(seq[:-1], seq[1:]) if v != p]
    assert runs == list(range(len(cells)))


def test_b3_box_gap_lower_bound():
    rng = np.random.default_rng(5)
    for _ in range(200):
        d = int(rng.integers(1, 4))
        P = rng.standard_normal((int(rng.integers(1, 9)), d)) + rng.uniform(-3, 3, d)
        Q = rng.standard_normal((int(rng.integers(1, 9)), d)) + rng.uniform(-3, 3, d)
        g2 = bs.gap2(P.min(0), P.max(0), Q.min(0), Q.max(0))
        C = ((P[:, None, :] - Q[None, :, :]) ** 2).sum(-1)
        assert g2 <= C.min() + 1e-12
        assert bs.pair_bound(np.zeros(d), np.zeros(d), P.min(0), P.max(0), Q.min(0),
                             Q.max(0)) == pytest.approx(-g2, abs=1e-12)
    p, q = rng.standard_normal(3), rng.standard_normal(3)
    assert bs.gap2(p, p, q, q) == pytest.approx(((p - q) ** 2).sum(), rel=1e-15)
    assert bs.gap2(np.zeros(2), np.ones(2), np.full(2, 0.5), np.full(2, 2.0)) == 0.0


def _grid_max1(u, v, a1, b1, a2, b2, k=401):
    x = np.linspace(a1, b1, k)[:, None]
    y = np.linspace(a2, b2, k)[None, :]
    return (u * x + v * y - (x - y) ** 2).max()


def test_b3_pair_bound_is_the_box_maximum():
    rng = np.random.default_rng(13)
    for _ in range(300):
        u, v = rng.normal(0, 2, 2)
        a1, a2 = rng.uniform(-1, 1, 2)
        b1, b2 = a1 + rng.uniform(0, 1.5), a2 + rng.uniform(0, 1.5)
        h = bs.hmax1(u, v, a1, b1, a2, b2)
        g = _grid_max1(u, v, a1, b1, a2, b2)
        # above every grid point, and within the grid's resolution of the top
        assert h >= g - 1e-12
        assert h <= g + 4 * (abs(u) + abs(v) + 8) * 1.5 / 400
    for _ in range(100):
        d = 3
        P = rng.standard_normal((6, d))
        Q = rng.standard_normal((5, d)) + 1.0
        u, v = rng.normal(0, 1, d), rng.normal(0, 1, d)
        H = bs.pair_bound(u, v, P.min(0), P.max(0), Q.min(0), Q.max(0))
        vals = P @ u[:, None] + (Q @ v)[None, :] - ((P[:, None] - Q[None]) ** 2).sum(-1)
        assert H >= vals.max() - 1e-12
    for _ in range(300):
        u, v = rng.normal(0, 2, 2)
        a1, a2 = rng.uniform(-1, 1, 2)
        b1, b2 = a1 + rng.uniform(0, 1.5), a2 + rng.uniform(0, 1.5)
        h = bs.bilinear_bound([u], [v], [a1], [b1], [a2], [b2])
        x = np.linspace(a1, b1, 201)[:, None]
        y = np.linspace(a2, b2, 201)[None, :]
        assert h == pytest.approx((u * x + v * y + 2 * x * y).max(), abs=1e-12)
    # one-point boxes: the bounds are the values themselves
    p, q = rng.standard_normal(3), rng.standard_normal(3)
    u, v = rng.normal(0, 1, 3), rng.normal(0, 1, 3)
    assert bs.bilinear_bound(u, v, p, p, q, q) == pytest.approx(u @ p + v @ q + 2 * p @ q,
                                                               abs=1e-12)
    u, v = rng.normal(0, 1, 3), rng.normal(0, 1, 3)
    assert bs.pair_bound(u, v, p, p, q, q) == pytest.approx(u @ p + v @ q - ((p - q) ** 2).sum(),
                                                           abs=1e-12)


def _clouds(seed, n, m, spread=1.0):
    rng = np.random.default_rng(seed)
    X = rng.uniform(0, 1, (n, 3)) * spread
    Y = (rng.uniform(0, 1, (m, 3)) * 0.8 + 0.1) * spread
    a = rng.standard_exponential(n)
    b = rng.standard_exponential(m)
    X = X[bs.morton_order(X)]
    Y = Y[bs.morton_order(Y)]
    return X, Y, a / a.sum(), b / b.sum()


def test_b4_delta_zero_is_dense():
    X, Y, a, b = _clouds(6, 700, 500)
    eps = 0.01
    rng = np.random.default_rng(7)
    g = rng.normal(0, 0.02, 500)
    f_cur = rng.normal(0, 0.02, 700)
    f_sp, lists = bs.f_update_sparse(X, Y, b, g, f_cur, eps, 0.0, BR=64, BK=32)
    assert all(len(l) == (500 + 31) // 32 for l in lists)
    f_ref = oracle.f_update(X, Y, b, g, eps)
    np.testing.assert_allclose(f_sp, f_ref, rtol=0, atol=1e-12)
    g_sp, _ = bs.g_update_sparse(X, Y, a, f_sp, g, eps, 0.0, BR=64, BK=32)
    np.testing.assert_allclose(g_sp, oracle.g_update(X, Y, a, f_sp, eps), rtol=0, atol=1e-12)


def _converged(X, Y, a, b, eps):
    r = oracle.sinkhorn(X, Y, a, b, eps=eps, iters=3000, tol=1e-9, check_every=10)
    return r["f"], r["g"]


def _block_mass_ok(R, K, w, pot_rows, pot_keys, eps, delta, BR, BK, chunk=0):
    """B5 check; returns the fraction of skipped (I, J) pairs."""
    lists = bs.screen(R, K, w, pot_rows, pot_keys, eps, delta, BR, BK, chunk=chunk)
    nbK = (len(K) + BK - 1) // BK
    skipped = 0
    for I, keep in enumerate(lists):
        rows = np.arange(I * BR, min((I + 1) * BR, len(R)))
        for J in set(range(nbK)) - set(keep.tolist()):
            skipped += 1
            keys = np.arange(J * BK, min((J + 1) * BK, len(K)))
            C = ((R[rows, None, :] - K[None, keys, :]) ** 2).sum(-1)
            mass = (w[keys][None, :] * np.exp((pot_rows[rows][:, None] + pot_keys[keys][None, :]
                                               - C) / eps)).sum(1)
            assert np.all(mass < delta / nbK * (1 + 1e-12)), (I, J, mass.max())
    return skipped / (len(lists) * nbK)


@pytest.mark.parametrize("delta", [1e-3, 1e-6])
def test_b5_skipped_block_mass(delta):
    X, Y, a, b = _clouds(8, 1500, 1200)
    eps = 2e-3
    f, g = _converged(X, Y, a, b, eps)
    # (at this size a block spans a good part of the cloud, so only some of
    # the pairs are far enough apart to be skipped)
    frac = _block_mass_ok(X, Y, b, f, g, eps, delta, 32, 32)
    assert frac > 0.1  # the check is not vacuous
    frac = _block_mass_ok(Y, X, a, g, f, eps, delta, 32, 32)
    assert frac > 0.1


@pytest.mark.parametrize("delta", [1e-3, 0.0])
def test_b5_two_level_screening(delta):
    """The two-level form (chunks of 4 blocks of 32 keys): every skipped
    block's true mass is still below delta / N_J (brute force), whole chunks
    are skipped, every block of a live chunk that the one-level screening
    keeps is kept, and delta = 0 keeps every block."""
    X, Y, a, b = _clouds(9, 800, 2400)
    eps = 1e-3
    f, g = _converged(X, Y, a, b, eps)
    frac = _block_mass_ok(X, Y, b, f, g, eps, delta, 32, 32, chunk=4)
    lists, beta, thr, cbeta = bs.screen(X, Y, b, f, g, eps, delta, 32, 32, return_bounds=True,
                                        chunk=4)
    flat = bs.screen(X, Y, b, f, g, eps, delta, 32, 32)
    nbK = (2400 + 31) // 32
    if delta == 0:
        assert frac == 0 and all(len(l) == nbK for l in lists)
        return
    assert frac > 0.3
    dead = cbeta < thr
    assert dead.mean() > 0.05  # chunks skipped whole, not only blocks
    for k, (keep, ref) in enumerate(zip(lists, flat)):
        assert set(keep.tolist()) <= set(ref.tolist()) | {int(np.argmax(beta[k]))}
        live_ref = [J for J in ref.tolist() if not dead[k, J // 4]]
        assert set(live_ref) <= set(keep.tolist())


@pytest.mark.parametrize("warm", [True, False])
def test_b6_certificate(warm):
    X, Y, a, b = _clouds(9, 1500, 1300)
    eps, delta = 2e-3, 1e-3
    if warm:
        f, g = _converged(X, Y, a, b, eps)
    else:
        rng = np.random.default_rng(10)
        f, g = rng.normal(0, 0.01, 1500), rng.normal(0, 0.01, 1300)
    f_sp, lists = bs.f_update_sparse(X, Y, b, g, f, eps, delta, BR=32, BK=32)
    kept = sum(len(l) for l in lists) / (len(lists) * ((1300 + 31) // 32))
    assert kept < 0.9
    f_ref = oracle.f_update(X, Y, b, g, eps)
    diff = f_sp - f_ref
    cert = bs.certificate(f_sp, f, eps, delta)
    assert np.all(diff >= -1e-12 * eps)
    assert np.all(diff <= cert + 1e-12 * eps)
    assert diff.max() > 0  # something was skipped
    if warm:  # near the fixed point the bound is about eps * delta
        assert cert.max() < 3 * eps * delta
    g_sp, _ = bs.g_update_sparse(X, Y, a, f_sp, g, eps, delta, BR=32, BK=32)
    g_ref = oracle.g_update(X, Y, a, f_sp, eps)
    cert = bs.certificate(g_sp, g, eps, delta)
    assert np.all(g_sp - g_ref >= -1e-12 * eps)
    assert np.all(g_sp - g_ref <= cert + 1e-12 * eps)


def test_b7_planted_slips_are_caught(monkeypatch):
    rng = np.random.default_rng(14)
    # a wrong sign in the edge maximiser undercuts the box maximum -> B3 fails
    bad = lambda u, v, a1, b1, a2, b2: max(
        [u * x + v * min(max(x - v / 2, a2), b2) - (x - min(max(x - v / 2, a2), b2)) ** 2
         for x in (a1, b1)] +
        [u * min(max(y - u / 2, a1), b1) + v * y - (min(max(y - u / 2, a1), b1) - y) ** 2
         for y in (a2, b2)])
    worst = 0.0
    for _ in range(100):
        u, v = rng.normal(0, 2, 2)
        a1, a2 = rng.uniform(-1, 1, 2)
        b1, b2 = a1 + rng.uniform(0, 1.5), a2 + rng.uniform(0, 1.5)
        worst = max(worst, _grid_max1(u, v, a1, b1, a2, b2) - bad(u, v, a1, b1, a2, b2))
    assert worst > 1e-3
    # the mean residual of the row fit instead of its maximum -> B5 fails
    X, Y, a, b = _clouds(11, 1200, 1000)
    eps, delta = 2e-3, 1e-3
    f, g = _converged(X, Y, a, b, eps)
    f = f + rng.normal(0, 20 * eps, len(f))
    _block_mass_ok(X, Y, b, f, g, eps, delta, 32, 32)  # the rule itself holds for any f
    orig_screen = bs.screen

    def screen_mean(R, K, w, pr, pk, eps_, delta_, BR=256, BK=32, return_bounds=False, chunk=0):
        assert chunk == 0
        lists, beta, thr = orig_screen(R, K, w, pr, pk, eps_, delta_, BR, BK, True)
        out = []
        for I in range(beta.shape[0]):
            P, fb = R[I * BR:(I + 1) * BR], pr[I * BR:(I + 1) * BR]
            r = fb - P @ bs.slope(P, fb)
            b2 = beta[I] - (r.max() - r.mean()) / eps_
            keep = np.nonzero(b2 >= thr)[0]
            out.append(keep if keep.size else np.array([int(np.argmax(b2))]))
        return out

    monkeypatch.setattr(bs, "screen", screen_mean)
    with pytest.raises(AssertionError):
        _block_mass_ok(X, Y, b, f, g, eps, delta, 32, 32)
