"""float64 oracle of the block-sparse (FlashSinkhorn 2 style) log-domain
Sinkhorn update on Morton-ordered low-dimensional point clouds.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): imported by
``tests/`` alone; the product path never imports it.  Plain numpy, written
for clarity; the dense cost is formed block by block, so it is meant for
small problems (a few thousand points).

Source: "FlashSinkhorn 2: block-sparse entropic optimal transport" (patty.io
explainer), sections on cutting space so that skipping is safe and on
guaranteeing the skip.  The page gives no formulas; the reading written out
here is:

* Morton order (section on cutting space): every coordinate c is quantised
  over the cloud's bounding box to B = floor(30 / d) bits,
      span_c = hi_c - lo_c,  scale_c = 2^B / span_c  (0 if span_c == 0),
      q_c = min(2^B - 1, floor((x_c - lo_c) * scale_c)),
  with every step a single float32 operation (subtraction, division,
  multiplication), and the code interleaves the bits: bit k of q_c becomes
  bit k*d + c of the code.  Points are ordered by code, ties by index.
* Blocks: consecutive runs of BR rows and of BK keys of the ordered clouds;
  each has an axis-aligned bounding box.  The squared box gap
      gap2(I, J) = sum_c max(0, lo_Jc - hi_Ic, lo_Ic - hi_Jc)^2
  bounds C_ij = |x_i - y_j|^2 from below for every pair of the two blocks.
* Screening (section on guaranteeing the skip): every block carries a
  linear fit of its potential, the least-squares slope
      u = (S_xx + lam I)^-1 S_xf,  S over the block's centred points and values,
      lam = 1e-6 trace(S_xx) (+1e-30),
  and, on the row side, the exact offset c_I = max_{i in I} (f_i - u_I.x_i),
  so that f_i <= c_I + u_I.x_i on the block (any slope would do; the fit
  only makes the bound tight).  On the key side the block mass
      G_J = log sum_{j in J} b_j exp((g_j - v_J.y_j) / eps).
  For i in I, j in J,
      f_i + g_j - C_ij <= c_I + (g_j - v_J.y_j) + H(I, J),
      H(I, J) = max_{x in box I, y in box J} (u_I.x + v_J.y - |x - y|^2),
  a concave quadratic that separates per coordinate; each 1-D maximum over
  a rectangle lies on one of its four edges, where it is a clipped stationary
  point.  So the mass key block J can contribute to row i, relative to the
  row's target a_i, is at most
      exp(beta(I, J)),  beta = c_I / eps + G_J + H(I, J) / eps.
  Block J is skipped for I when beta < log(delta / N_J) (N_J = number of key
  blocks), so that the skipped mass of every row stays below delta * a_i; if
  every block of I would be skipped, the one with the largest bound is kept.
  With zero slopes H is minus the squared box gap
      gap2(I, J) = sum_c max(0, lo_Jc - hi_Ic, lo_Ic - hi_Jc)^2.
  A second bound of the same form comes from the dot-product split of the
  exponent, f_i + g_j - C_ij = phi_i + psi_j + 2 x_i.y_j with phi_i =
  f_i - |x_i|^2, psi_j = g_j - |y_j|^2: the same fits and offsets taken of
  phi and psi, and
      H2(I, J) = max over the two boxes of (u2_I.x + v2_J.y + 2 x.y),
  a bilinear function per coordinate, whose maximum over a rectangle is at a
  corner.  The first form is tight where f is nearly linear over a block
  (little displacement), the second where phi is (a map that concentrates
  mass); beta is the smaller of the two bounds.
  The same rule with the roles of the clouds swapped screens the g-update
  (per column).
* Retained-block update: f_i = -eps log sum over the kept blocks' keys of
  b_j exp((g_j - C_ij) / eps).  Skipping only removes positive terms, so
      0 <= f_sparse_i - f_dense_i <= eps * log(1 + delta * exp((f_sparse_i - f_i) / eps))
  with f_i the potential being replaced (the certificate below).

Pins (tests/test_oracle_blocksparse.py): bit interleaving against a
recursive Z-order enumeration; quantisation endpoints, monotonicity and the
degenerate axis; the box gap, H and H2 against brute-force maxima over the
blocks' points and a fine grid of the boxes; delta = 0 against the dense
oracle update; the per-block mass bound against brute force on every
skipped block; the certificate against the dense update.
"""
from __future__ import annotations

import numpy as np

CODE_BITS = 30


def morton_bits(d: int) -> int:
    """Bits per coordinate of the Morton code (B = floor(30 / d))."""
    if not 1 <= d <= 30:
        raise ValueError("d must be in [1, 30]")
    return CODE_BITS // d


def quantize(X) -> np.ndarray:
    """Integer cell coordinates q (n x d, int64) of the points over the
    cloud's bounding box, every step in float32 as stated in the header."""
    X32 = np.asarray(X, np.float32)
    n, d = X32.shape
    B = morton_bits(d)
    lo = X32.min(axis=0)
    hi = X32.max(axis=0)
    span = (hi - lo).astype(np.float32)
    top = np.float32(2.0 ** B)
    scale = np.zeros(d, np.float32)
    for c in range(d):
        if span[c] > 0:
            scale[c] = np.float32(top / span[c])
    t = (X32 - lo).astype(np.float32) * scale
    q = np.floor(t.astype(np.float64)).astype(np.int64)
    return np.clip(q, 0, (1 << B) - 1)


def interleave(q, d: int) -> np.ndarray:
    """Morton code of integer cell coordinates: bit k of q[:, c] -> bit k*d + c."""
    q = np.asarray(q, np.int64).reshape(-1, d)
    B = morton_bits(d)
    code = np.zeros(q.shape[0], np.int64)
    for k in range(B):
        for c in range(d):
            code |= ((q[:, c] >> k) & 1) << (k * d + c)
    return code


def morton_codes(X) -> np.ndarray:
    X = np.asarray(X, np.float32)
    return interleave(quantize(X), X.shape[1])


def morton_order(X) -> np.ndarray:
    """Permutation that sorts the points by Morton code, ties by index."""
    return np.argsort(morton_codes(X), kind="stable")


def block_boxes(P, B: int):
    """(lo, hi) per block of B consecutive points (the last may be short)."""
    P = np.asarray(P, np.float64)
    nb = (P.shape[0] + B - 1) // B
    lo = np.stack([P[k * B:(k + 1) * B].min(axis=0) for k in range(nb)])
    hi = np.stack([P[k * B:(k + 1) * B].max(axis=0) for k in range(nb)])
    return lo, hi


def gap2(lo1, hi1, lo2, hi2) -> float:
    """Squared distance between two axis-aligned boxes (0 if they overlap)."""
    g = np.maximum(0.0, np.maximum(np.asarray(lo2) - np.asarray(hi1),
                                   np.asarray(lo1) - np.asarray(hi2)))
    return float((g * g).sum())


def _lse(v) -> float:
    v = np.asarray(v, np.float64)
    m = v.max()
    if not np.isfinite(m):
        return float(m)
    return float(m + np.log(np.exp(v - m).sum()))


def slope(P, v) -> np.ndarray:
    """Regularised least-squares slope of the values v over the points P."""
    P, v = np.asarray(P, np.float64), np.asarray(v, np.float64)
    Pc = P - P.mean(axis=0)
    vc = v - v.mean()
    S = Pc.T @ Pc
    lam = 1e-6 * np.trace(S) + 1e-30
    return np.linalg.solve(S + lam * np.eye(P.shape[1]), Pc.T @ vc)


def hmax1(u: float, v: float, a1: float, b1: float, a2: float, b2: float) -> float:
    """max of u x + v y - (x - y)^2 over x in [a1, b1], y in [a2, b2]."""
    h = lambda x, y: u * x + v * y - (x - y) ** 2
    cands = []
    for x in (a1, b1):
        cands.append(h(x, min(max(x + v / 2, a2), b2)))
    for y in (a2, b2):
        cands.append(h(min(max(y + u / 2, a1), b1), y))
    return max(cands)


def pair_bound(u, v, lo1, hi1, lo2, hi2) -> float:
    """H = max over the box pair of u.x + v.y - |x - y|^2 (sum of 1-D maxima)."""
    return float(sum(hmax1(u[c], v[c], lo1[c], hi1[c], lo2[c], hi2[c]) for c in range(len(u))))


def bilinear_bound(u, v, lo1, hi1, lo2, hi2) -> float:
    """H2 = max over the box pair of u.x + v.y + 2 x.y (corners, per coordinate)."""
    tot = 0.0
    for c in range(len(u)):
        tot += max(u[c] * x + v[c] * y + 2.0 * x * y for x in (lo1[c], hi1[c])
                   for y in (lo2[c], hi2[c]))
    return float(tot)


def _key_group_fits(K, w_keys, pot_keys, eps, size):
    """Per group of `size` consecutive keys: slopes and log-sum-exp terms of
    both forms (g and g - |y|^2), as for a key block."""
    V, G, V2, G2 = [], [], [], []
    for J in range((K.shape[0] + size - 1) // size):
        Q, g, w = K[J * size:(J + 1) * size], pot_keys[J * size:(J + 1) * size], \
            w_keys[J * size:(J + 1) * size]
        psi = g - (Q * Q).sum(axis=1)
        V.append(slope(Q, g))
        G.append(_lse(np.log(w) + (g - Q @ V[-1]) / eps))
        V2.append(slope(Q, psi))
        G2.append(_lse(np.log(w) + (psi - Q @ V2[-1]) / eps))
    return V, G, V2, G2


def screen(R, K, w_keys, pot_rows, pot_keys, eps: float, delta: float, BR: int = 256,
           BK: int = 32, return_bounds: bool = False, row_blocks=None, chunk: int = 0):
    """Kept key blocks (ascending indices) of every row block, for the update
    of the rows' potential from the keys' potential (see the header).
    With return_bounds, also the log bound matrix beta[I, J] and the log
    threshold (and, with chunks, the chunk bound matrix).  row_blocks: screen
    only these row blocks (lists and rows of beta in that order).

    chunk > 0: two-level screening.  Chunks of `chunk` consecutive key blocks
    get a bound of their own (the same two forms over the chunk's box and
    keys); a chunk whose bound is below the threshold is skipped whole, since
    each of its blocks holds at most the chunk's mass.  Only the blocks of the
    other chunks, and always those of the chunk of largest bound, are
    screened one by one; the fallback block is the best of those."""
    R, K = np.asarray(R, np.float64), np.asarray(K, np.float64)
    w_keys = np.asarray(w_keys, np.float64)
    pot_rows = np.asarray(pot_rows, np.float64)
    pot_keys = np.asarray(pot_keys, np.float64)
    rlo, rhi = block_boxes(R, BR)
    klo, khi = block_boxes(K, BK)
    nbK = klo.shape[0]
    blocks = list(range(rlo.shape[0])) if row_blocks is None else [int(I) for I in row_blocks]
    nbR = len(blocks)
    U, c, U2, c2 = [], [], [], []
    for I in blocks:
        P, f = R[I * BR:(I + 1) * BR], pot_rows[I * BR:(I + 1) * BR]
        phi = f - (P * P).sum(axis=1)
        U.append(slope(P, f))
        c.append((f - P @ U[-1]).max())
        U2.append(slope(P, phi))
        c2.append((phi - P @ U2[-1]).max())
    V, G, V2, G2 = _key_group_fits(K, w_keys, pot_keys, eps, BK)
    thr = np.log(delta / nbK) if delta > 0 else -np.inf
    beta = np.empty((nbR, nbK))

    def bound(k, I, u, gg, u2, gg2, lo, hi):
        H = pair_bound(U[k], u, rlo[I], rhi[I], lo, hi)
        H2 = bilinear_bound(U2[k], u2, rlo[I], rhi[I], lo, hi)
        return min(c[k] / eps + gg + H / eps, c2[k] / eps + gg2 + H2 / eps)

    if chunk > 0:
        nbC = (nbK + chunk - 1) // chunk
        clo, chi = block_boxes(K, BK * chunk)
        CV, CG, CV2, CG2 = _key_group_fits(K, w_keys, pot_keys, eps, BK * chunk)
        cbeta = np.array([[bound(k, I, CV[C], CG[C], CV2[C], CG2[C], clo[C], chi[C])
                           for C in range(nbC)] for k, I in enumerate(blocks)])
    lists = []
    for k, I in enumerate(blocks):
        if chunk > 0:
            live = cbeta[k] >= thr
            live[int(np.argmax(cbeta[k]))] = True
        for J in range(nbK):
            if chunk > 0 and not live[J // chunk]:
                beta[k, J] = -np.inf  # not screened
                continue
            beta[k, J] = bound(k, I, V[J], G[J], V2[J], G2[J], klo[J], khi[J])
        keep = np.nonzero(beta[k] >= thr)[0]
        if keep.size == 0:
            keep = np.array([int(np.argmax(beta[k]))])
        lists.append(keep)
    if return_bounds:
        return (lists, beta, thr, cbeta) if chunk > 0 else (lists, beta, thr)
    return lists


def update_sparse(R, K, w_keys, pot_keys, pot_rows, eps: float, delta: float, BR: int = 256,
                  BK: int = 32, row_blocks=None, chunk: int = 0):
    """Retained-block update of the rows' potential; returns (new, lists).
    row_blocks: update only these row blocks (the other entries are NaN)."""
    R, K = np.asarray(R, np.float64), np.asarray(K, np.float64)
    w_keys = np.asarray(w_keys, np.float64)
    pot_keys = np.asarray(pot_keys, np.float64)
    lists = screen(R, K, w_keys, pot_rows, pot_keys, eps, delta, BR, BK, row_blocks=row_blocks,
                   chunk=chunk)
    blocks = range(len(lists)) if row_blocks is None else [int(I) for I in row_blocks]
    out = np.full(R.shape[0], np.nan)
    for I, keep in zip(blocks, lists):
        rows = np.arange(I * BR, min((I + 1) * BR, R.shape[0]))
        keys = np.concatenate([np.arange(J * BK, min((J + 1) * BK, K.shape[0])) for J in keep])
        C = ((R[rows, None, :] - K[None, keys, :]) ** 2).sum(-1)
        z = np.log(w_keys[keys])[None, :] + (pot_keys[keys][None, :] - C) / eps
        m = z.max(axis=1)
        out[rows] = -eps * (m + np.log(np.exp(z - m[:, None]).sum(axis=1)))
    return out, lists


def f_update_sparse(X, Y, b, g, f_cur, eps: float, delta: float, BR: int = 256, BK: int = 32):
    return update_sparse(X, Y, b, g, f_cur, eps, delta, BR, BK)


def g_update_sparse(X, Y, a, f, g_cur, eps: float, delta: float, BR: int = 256, BK: int = 32):
    return update_sparse(Y, X, a, f, g_cur, eps, delta, BR, BK)


def certificate(new, cur, eps: float, delta: float) -> np.ndarray:
    """Upper bound on new_sparse - new_dense per row (see the header)."""
    new, cur = np.asarray(new, np.float64), np.asarray(cur, np.float64)
    return eps * np.log1p(delta * np.exp((new - cur) / eps))


def sinkhorn_sparse(X, Y, a, b, eps: float, iters: int, delta: float, f0=None, g0=None,
                    BR: int = 256, BK: int = 32):
    """Alternating retained-block updates (f from g, then g from the new f)."""
    f = np.zeros(len(X)) if f0 is None else np.array(f0, np.float64)
    g = np.zeros(len(Y)) if g0 is None else np.array(g0, np.float64)
    for _ in range(iters):
        f, _l = f_update_sparse(X, Y, b, g, f, eps, delta, BR, BK)
        g, _l = g_update_sparse(X, Y, a, f, g, eps, delta, BR, BK)
    return f, g
