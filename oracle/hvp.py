"""float64 dense oracle of the Hessian-vector product of the entropic OT loss
with respect to the row cloud X (squared-Euclidean cost).

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): imported by
``tests/`` alone; the product path never imports it.  Plain numpy on the
dense n x m plan, so it is meant for small problems.

Source: "FlashSinkhorn" explainer, section "Method", part 3, states that
Hessian-vector products are evaluated as a sequence of transport-vector and
transport-matrix products, without the Hessian or the plan in memory; the
pages print no formula.  The reading written out here (implicit
differentiation through the Sinkhorn fixed point):

  loss L(X) = OT_eps at the optimal potentials (f*, g*)(X); its gradient is
      G_i = 2 sum_j P_ij (x_i - y_j),  P_ij = a_i b_j exp((f_i+g_j-C_ij)/eps),
  the envelope theorem (pinned against finite differences of the converged
  loss by the gradient tests).  For a direction V (n x d), differentiating G
  along X + tV with the potentials moving so that both marginals of P stay
  fixed:
      dC_ij = 2 (x_i - y_j).v_i,
      dP_ij = P_ij (df_i + dg_j - dC_ij) / eps,
      sum_j dP_ij = 0, sum_i dP_ij = 0, i.e.
      [diag(r)  P      ] [df]   [u]      u_i = sum_j P_ij dC_ij,
      [P^T      diag(c)] [dg] = [w],     w_j = sum_i P_ij dC_ij,
  with r = P 1, c = P^T 1 (the marginals; a and b at convergence).  The
  system is singular along (1, -1), which leaves dP unchanged; its
  minimum-norm least-squares solution is taken.  Then
      (H V)_i = 2 r_i v_i + 2 sum_j dP_ij (x_i - y_j).
  Evaluated at any (f, g) by treating their plan as the optimum (r, c in
  place of a, b).

Pins (tests/test_oracle_hvp.py): central finite differences of the gradient
at re-converged potentials (independent of the derivation), symmetry
<U, H V> = <V, H U>, and the single-target closed form H V = 2 a V.
"""
from __future__ import annotations

import numpy as np


def plan(X, Y, a, b, f, g, eps):
    """Dense P_ij = a_i b_j exp((f_i + g_j - |x_i - y_j|^2) / eps), float64."""
    X, Y = np.asarray(X, np.float64), np.asarray(Y, np.float64)
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    f, g = np.asarray(f, np.float64), np.asarray(g, np.float64)
    C = ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)
    return np.exp(np.log(a)[:, None] + np.log(b)[None, :] + (f[:, None] + g[None, :] - C) / eps)


def hvp(X, Y, a, b, f, g, V, eps, return_parts=False, P=None):
    """(H V) of the entropic OT loss with respect to X, at the plan of (f, g)
    (or at a given dense plan P, with the cost derivative still taken from X
    and Y: the form a solver whose scores round the points differentiates)."""
    X, Y, V = (np.asarray(t, np.float64) for t in (X, Y, V))
    n = X.shape[0]
    P = plan(X, Y, a, b, f, g, eps) if P is None else np.asarray(P, np.float64)
    r, c = P.sum(1), P.sum(0)
    D = X[:, None, :] - Y[None, :, :]            # x_i - y_j, n x m x d
    dC = 2.0 * np.einsum("ijk,ik->ij", D, V)      # n x m
    u, w = (P * dC).sum(1), (P * dC).sum(0)
    A = np.block([[np.diag(r), P], [P.T, np.diag(c)]])
    sol = np.linalg.lstsq(A, np.concatenate([u, w]), rcond=None)[0]
    df, dg = sol[:n], sol[n:]
    dP = P * (df[:, None] + dg[None, :] - dC) / eps
    HV = 2.0 * r[:, None] * V + 2.0 * np.einsum("ij,ijk->ik", dP, D)
    if return_parts:
        return HV, {"df": df, "dg": dg, "r": r, "c": c}
    return HV
