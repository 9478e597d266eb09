"""Shared helpers of the GPU tests: run the HIP solver, run the oracle, and
reproduce on the CPU the centring and operand rounding that the bf16/fp16
paths apply (independent numpy code; nothing here is shared with the
library)."""
from __future__ import annotations

import numpy as np

import oracle


def dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def centres(X: np.ndarray, Y: np.ndarray):
    """Midpoint of each cloud's own bounding box, in float32 arithmetic."""
    def mid(P):
        P = np.asarray(P, dtype=np.float32)
        return ((P.min(0) + P.max(0)) * np.float32(0.5)).astype(np.float32)

    return mid(X), mid(Y)


def normalise_rows(P) -> np.ndarray:
    """The cosine cost's points as the library forms them: each row times
    float32(1 / sqrt(float32 sum of squares)), in float32."""
    P = np.asarray(P, dtype=np.float32)
    s = np.sum(P.astype(np.float64) ** 2, axis=1)
    inv = (1.0 / np.sqrt(s.astype(np.float32))).astype(np.float32)
    return (P * inv[:, None]).astype(np.float32)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def round_f16(x32: np.ndarray) -> np.ndarray:
    return np.asarray(x32, dtype=np.float32).astype(np.float16).astype(np.float32)


class RoundedProblem:
    """The problem a score path solves, written as an oracle problem.

    The path centres each cloud on its own bounding-box midpoint (nu for X,
    mu for Y), rounds x' = x - nu and y' = y - mu (fp32 subtraction, then
    bf16 / fp16 rounding; prec "fp32" keeps the fp32 difference), and
    evaluates
        C~_ij = A_i + B_j - 2 xr_i . yr_j,
        A_i = |x_i - mu|^2 - |nu - mu|^2 / 2,  B_j = |y_j - nu|^2 - |nu - mu|^2 / 2
    with A, B from the unrounded points.  Since C~_ij = |xr_i - yr_j|^2 +
    alpha_i + beta_j with alpha_i = A_i - |xr_i|^2 and beta_j = B_j - |yr_j|^2,
    the potentials of C~ are those of the rounded clouds (xr, yr) shifted by
    alpha, beta:  f = f_r + alpha,  g = g_r + beta.  The oracle then runs on
    plain points, unchanged."""

    def __init__(self, X, Y, prec: str):
        nu, mu = centres(X, Y)
        r = {"bf16": round_bf16, "fp16": round_f16, "fp32": lambda v: v}[prec]
        X32 = np.asarray(X, dtype=np.float32)
        Y32 = np.asarray(Y, dtype=np.float32)
        self.Xr = r(X32 - nu).astype(np.float64)
        self.Yr = r(Y32 - mu).astype(np.float64)
        dl = nu.astype(np.float64) - mu.astype(np.float64)
        h = 0.5 * float(dl @ dl)
        A = np.sum((X32.astype(np.float64) - mu) ** 2, axis=1) - h
        B = np.sum((Y32.astype(np.float64) - nu) ** 2, axis=1) - h
        self.alpha = A - np.sum(self.Xr ** 2, axis=1)
        self.beta = B - np.sum(self.Yr ** 2, axis=1)

    def solve(self, a, b, **kw):
        """oracle.sinkhorn from g = 0 on C~ (g_r starts at -beta)."""
        out = oracle.sinkhorn(self.Xr, self.Yr, a, b, g0=-self.beta, **kw)
        return {"f": out["f"] + self.alpha, "g": out["g"] + self.beta}

    def f_update_rows(self, b, g, eps, rows):
        rows = np.asarray(rows)
        return oracle.f_update_rows(self.Xr, self.Yr, b, np.asarray(g) - self.beta, eps,
                                    rows) + self.alpha[rows]

    def g_update_cols(self, a, f, eps, cols):
        cols = np.asarray(cols)
        return oracle.g_update_cols(self.Xr, self.Yr, a, np.asarray(f) - self.alpha, eps,
                                    cols) + self.beta[cols]

    def transport(self, a, b, f, g, V, eps, divide_by_a=False, rows=None):
        return oracle.transport(self.Xr, self.Yr, a, b, np.asarray(f) - self.alpha,
                                np.asarray(g) - self.beta, V, eps, divide_by_a=divide_by_a,
                                rows=rows)


def gpu_solve(X, Y, a, b, *, eps, iters, prec="auto", n_stages=1, eps_start=None, tol=0.0,
              check_every=10, dv_max=0, cost="sqeuclidean"):
    from streaming_sinkhorn_solver_amd import binding

    Xd, Yd, ad, bd = dev(X), dev(Y), dev(a), dev(b)
    p, f, g, info = binding.solve(Xd, Yd, ad, bd, eps=eps, iters=iters, prec=prec,
                                  n_stages=n_stages, eps_start=eps_start, tol=tol,
                                  check_every=check_every, dv_max=dv_max, cost=cost)
    import torch

    torch.cuda.synchronize()
    return p, f, g, info, (Xd, Yd, ad, bd)


def max_err(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64))))


def oracle_solve(X, Y, a, b, *, eps, iters, n_stages=1, eps_start=None):
    return oracle.sinkhorn(X, Y, a, b, eps=eps, iters=iters, n_stages=n_stages,
                           eps_start=eps_start)
