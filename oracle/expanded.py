"""float64 Sinkhorn with the cost matrix formed by a library matrix product.

TEST INFRASTRUCTURE ONLY: used by the script that writes the stored
expected values of the large recipes (``tests/golden/make_golden_full.py``)
and by its pins in ``tests/test_oracle_expanded.py``; the product path never
imports it.  It shares no code with the HIP library.

Why it exists: the direct-difference oracle (``oracle.c``) evaluates every
|x_i - y_j|^2 coordinate by coordinate.  That is the plainest form, but at
50,000 x 50,000 points in 512 dimensions one half-step costs it minutes of
CPU time per core group, and the annealed 1024-D recipe needs 400 of them.
Here the same update is evaluated through the identity

    |x_i - y_j|^2 = |x_i|^2 + |y_j|^2 - 2 x_i . y_j,

which the FlashSinkhorn explainer ("FlashSinkhorn: IO-Aware Entropic Optimal
Transport on GPU", section "Method", part 1) uses to recast the update as a
row-wise log-sum-exp of dot-product scores:

    f_i <- -eps * LSE_j [ (g_j - C_ij)/eps + log b_j ]      (f-update)
         = |x_i|^2 - eps * LSE_j [ (2/eps) x_i.y_j + (g_j - |y_j|^2)/eps + log b_j ]
    g_j <- -eps * LSE_i [ (f_i - C_ij)/eps + log a_i ]      (g-update, new f)

The dot products come from one float64 matrix product with the per-column
term added in the same library call (torch.addmm), the log-sum-exp from the
library's two-pass float64 routine (maximum, then the sum of exponentials).
It follows the same readings as ``oracle.c``: alternating order, g starting at 0,
no 1/2 in the cost, annealed stages eps_s = eps0 (eps_end/eps0)^(s/(S-1))
with the potentials carried over (the stage values come from ``oracle.c``).
Rows are processed in groups only to bound the memory of the n x m score
block; every row's update is independent of the others, so the grouping
changes no arithmetic.

In float64 the expansion's cancellation error is about 1e-16 (|x|^2 + |y|^2)
per entry, some 1e-13 of eps for every recipe here, far below every parity
bar.  Pinned against the direct-difference oracle iterate for iterate on
every recipe's distribution at reduced size and, at full size, on sampled
rows and columns of the written iterates (``tests/test_oracle_expanded.py``,
``tests/golden/make_golden_full.py``).
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np
import torch

from . import stage_eps

__all__ = ["f_update", "g_update", "sinkhorn"]

_ROWS_PER_GROUP = 2048


def _soft_min(P: torch.Tensor, pn: torch.Tensor, Q: torch.Tensor, qn: torch.Tensor,
              logw: torch.Tensor, pot: torch.Tensor, eps: float) -> torch.Tensor:
    """out_i = -eps LSE_k[(pot_k - C(p_i, q_k))/eps + log w_k] with C expanded:
    the argument is beta_k + (2/eps) p_i.q_k - |p_i|^2/eps, beta_k =
    (pot_k - |q_k|^2)/eps + log w_k, and the row term leaves the LSE."""
    beta = (pot - qn) / eps + logw
    out = torch.empty(P.shape[0], dtype=torch.float64)
    for r0 in range(0, P.shape[0], _ROWS_PER_GROUP):
        r1 = min(P.shape[0], r0 + _ROWS_PER_GROUP)
        z = torch.addmm(beta.expand(r1 - r0, -1), P[r0:r1], Q.T, beta=1.0, alpha=2.0 / eps)
        out[r0:r1] = pn[r0:r1] - eps * torch.logsumexp(z, dim=1)
    return out


class _Problem:
    """float64 copies of the clouds, their squared norms and log-weights."""

    def __init__(self, X, Y, a, b):
        self.X = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float64))
        self.Y = torch.from_numpy(np.ascontiguousarray(Y, dtype=np.float64))
        self.xn = (self.X * self.X).sum(dim=1)
        self.yn = (self.Y * self.Y).sum(dim=1)
        self.la = torch.log(torch.from_numpy(np.asarray(a, dtype=np.float64)))
        self.lb = torch.log(torch.from_numpy(np.asarray(b, dtype=np.float64)))

    def f_update(self, g: torch.Tensor, eps: float) -> torch.Tensor:
        return _soft_min(self.X, self.xn, self.Y, self.yn, self.lb, g, eps)

    def g_update(self, f: torch.Tensor, eps: float) -> torch.Tensor:
        return _soft_min(self.Y, self.yn, self.X, self.xn, self.la, f, eps)


def f_update(X, Y, b, g, eps: float) -> np.ndarray:
    """The f-update of every row (a is not needed; pass ones)."""
    p = _Problem(X, Y, np.ones(len(X)), b)
    return p.f_update(torch.from_numpy(np.asarray(g, dtype=np.float64)), eps).numpy()


def g_update(X, Y, a, f, eps: float) -> np.ndarray:
    """The g-update of every column."""
    p = _Problem(X, Y, a, np.ones(len(Y)))
    return p.g_update(torch.from_numpy(np.asarray(f, dtype=np.float64)), eps).numpy()


def sinkhorn(X, Y, a, b, *, eps: float, iters: int, n_stages: int = 1,
             eps_start: Optional[float] = None,
             on_iteration: Optional[Callable[[int, float, np.ndarray, np.ndarray], None]] = None):
    """Alternating iteration from g = 0: ``n_stages`` stages of ``iters``
    iterations each (f-update, then g-update with the new f).  Returns a
    dict with f, g (float64) and the number of iterations.  ``on_iteration``
    (if given) is called after every iteration with (iteration, eps, f, g)."""
    p = _Problem(X, Y, a, b)
    f = torch.zeros(p.X.shape[0], dtype=torch.float64)
    g = torch.zeros(p.Y.shape[0], dtype=torch.float64)
    e0 = eps if eps_start is None else eps_start
    done = 0
    for s in range(n_stages):
        e = stage_eps(s, n_stages, e0, eps)
        for _ in range(iters):
            f = p.f_update(g, e)
            g = p.g_update(f, e)
            done += 1
            if on_iteration is not None:
                on_iteration(done, e, f.numpy(), g.numpy())
    return {"f": f.numpy().copy(), "g": g.numpy().copy(), "iters": done}
