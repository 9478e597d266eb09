"""Shared helpers of the GPU tests: run the HIP solver, run the oracle, and
reproduce on the CPU the operand rounding that the bf16/fp16 paths apply
(independent numpy code; nothing here is shared with the library)."""
from __future__ import annotations

import numpy as np

import oracle


def dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def bbox_shift(X: np.ndarray, Y: np.ndarray) -> np.ndarray:
    """Midpoint of the joint bounding box, in float32 arithmetic."""
    mn = np.minimum(X.min(0), Y.min(0)).astype(np.float32)
    mx = np.maximum(X.max(0), Y.max(0)).astype(np.float32)
    return ((mn + mx) * np.float32(0.5)).astype(np.float32)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def round_f16(x32: np.ndarray) -> np.ndarray:
    return np.asarray(x32, dtype=np.float32).astype(np.float16).astype(np.float32)


def rounded_operands(X, Y, prec: str):
    """The points the bf16/fp16 paths actually solve with (shifted, rounded)."""
    s = bbox_shift(X, Y)
    Xs = (X.astype(np.float32) - s).astype(np.float32)
    Ys = (Y.astype(np.float32) - s).astype(np.float32)
    r = round_bf16 if prec == "bf16" else round_f16
    return r(Xs), r(Ys)


def gpu_solve(X, Y, a, b, *, eps, iters, prec="auto", n_stages=1, eps_start=None, tol=0.0,
              check_every=10, dv_max=0):
    from streaming_sinkhorn_solver_amd import binding

    Xd, Yd, ad, bd = dev(X), dev(Y), dev(a), dev(b)
    p, f, g, info = binding.solve(Xd, Yd, ad, bd, eps=eps, iters=iters, prec=prec,
                                  n_stages=n_stages, eps_start=eps_start, tol=tol,
                                  check_every=check_every, dv_max=dv_max)
    import torch

    torch.cuda.synchronize()
    return p, f, g, info, (Xd, Yd, ad, bd)


def max_err(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64))))


def oracle_solve(X, Y, a, b, *, eps, iters, n_stages=1, eps_start=None):
    return oracle.sinkhorn(X, Y, a, b, eps=eps, iters=iters, n_stages=n_stages,
                           eps_start=eps_start)
