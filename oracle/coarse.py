"""float64 oracle of the coarse (centroid) stage of the block-sparse form:
centroids of cells, the lift of their potentials to the points, and the
sampled marginal check.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): imported by
``tests/`` alone; the product path never imports it.  Plain numpy.

Source: "FlashSinkhorn 2: block-sparse entropic optimal transport" (patty.io
explainer), sections on solving at a coarse resolution first and on trusting
the lifted solution.  The page gives no formulas; the reading written out
here:

* cells are runs of `cell` consecutive points of a Morton-ordered cloud (the
  last may be shorter); a cell's centroid is the weighted mean of its points
  and its weight the sum of theirs;
* the coarse problem is the transport between the two centroid clouds with
  those weights, solved by the ordinary Sinkhorn iteration;
* the lift gives every point its cell's potential as it is;
* the check draws sampled rows S and columns T and computes their exact
  marginals under the lifted potentials,
      err_rows = sum_{i in S} |r_i - a_i| / sum_{i in S} a_i,
      r_i = a_i sum_j b_j exp((f_i + g_j - C_ij) / eps),
  and err_cols the same for columns; the lift is accepted when both are at
  most the tolerance, else the coarse iteration continues and the check is
  repeated.

Pins (tests/test_oracle_coarse.py): centroid sums (weight and first moment)
conserved; one-point cells reproduce the fine problem (lift = identity,
coarse potentials = fine potentials); the sampled check over all rows and
columns equals the full L1 marginal residual divided by the total mass; a
cell holding copies of one point has that point as centroid.
"""
from __future__ import annotations

import numpy as np

import oracle


def centroids(P, w, cell: int):
    """(C, W): weighted means and weight sums of runs of `cell` points."""
    P, w = np.asarray(P, np.float64), np.asarray(w, np.float64)
    nc = (len(P) + cell - 1) // cell
    C = np.empty((nc, P.shape[1]))
    W = np.empty(nc)
    for k in range(nc):
        ww = w[k * cell:(k + 1) * cell]
        W[k] = ww.sum()
        C[k] = (ww[:, None] * P[k * cell:(k + 1) * cell]).sum(axis=0) / W[k]
    return C, W


def lift(F, n: int, cell: int) -> np.ndarray:
    """f_i = F[i // cell]."""
    F = np.asarray(F, np.float64)
    return F[np.arange(n) // cell]


def sampled_marginal_error(X, Y, a, b, f, g, eps: float, rows, cols):
    """(err_rows, err_cols) over the sampled rows and columns."""
    X, Y = np.asarray(X, np.float64), np.asarray(Y, np.float64)
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    f, g = np.asarray(f, np.float64), np.asarray(g, np.float64)
    rows, cols = np.asarray(rows), np.asarray(cols)
    C = ((X[rows, None, :] - Y[None, :, :]) ** 2).sum(-1)
    r = a[rows] * (b[None, :] * np.exp((f[rows, None] + g[None, :] - C) / eps)).sum(axis=1)
    Cc = ((X[:, None, :] - Y[None, cols, :]) ** 2).sum(-1)
    c = b[cols] * (a[:, None] * np.exp((f[:, None] + g[None, cols] - Cc) / eps)).sum(axis=0)
    return (float(np.abs(r - a[rows]).sum() / a[rows].sum()),
            float(np.abs(c - b[cols]).sum() / b[cols].sum()))


def coarse_start(X, Y, a, b, cell: int, eps: float, iters: int, n_stages: int = 1,
                 eps_start=None, more_iters: int = 10, tol: float = 1e-2, max_rounds: int = 5,
                 rows=None, cols=None):
    """The coarse stage: solve on centroids, lift, check, continue until the
    check passes or max_rounds checks were made.  Returns a dict with the
    lifted (f, g), the coarse (F, G), the rounds and the last errors."""
    CX, WX = centroids(X, a, cell)
    CY, WY = centroids(Y, b, cell)
    r = oracle.sinkhorn(CX, CY, WX, WY, eps=eps, iters=iters, n_stages=n_stages,
                        eps_start=eps_start)
    F, G = r["f"], r["g"]
    rows = np.arange(len(X)) if rows is None else rows
    cols = np.arange(len(Y)) if cols is None else cols
    for k in range(max_rounds):
        f, g = lift(F, len(X), cell), lift(G, len(Y), cell)
        err = sampled_marginal_error(X, Y, a, b, f, g, eps, rows, cols)
        if max(err) <= tol or k == max_rounds - 1:
            return {"f": f, "g": g, "F": F, "G": G, "rounds": k + 1, "errors": err,
                    "accepted": max(err) <= tol}
        r = oracle.sinkhorn(CX, CY, WX, WY, eps=eps, iters=more_iters, g0=G)
        F, G = r["f"], r["g"]
