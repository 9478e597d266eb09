"""Seeded synthetic inputs for the streaming Sinkhorn solver.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle.  It draws point clouds, weights and transport right-hand sides and
holds none of the solver's arithmetic: no cost, no log-sum-exp, no potential
update, no epsilon schedule evaluation.  Everything is drawn in float64 from
``numpy.random.default_rng(seed)`` (PCG64) in a fixed order and cast once to
float32, so both sides receive identical bytes.

The pages (FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU, section
"Experimental results") measure on synthetic point clouds whose distributions
they do not describe; the five recipes below stand in for them:

* ``c1`` 512 x 512 points in 3-D, two unit Gaussians offset by 0.5, uniform
  weights, eps 0.1, 100 alternating iterations.
* ``c2`` 10k x 10k points in 64-D, isotropic Gaussians of variance 1/d and
  0.5/d around a random mean, uniform weights, eps 0.05, 200 iterations.
* ``c3`` 50k x 50k points in 512-D, two independent 10-component Gaussian
  mixtures (means N(0, I/d), component std 0.3/sqrt(d)), Dirichlet(1)
  weights, eps 0.1, 100 iterations, then the barycentric projection P.Y / a.
* ``c4`` 50k x 30k points in 1024-D, X uniform on the unit sphere, Y
  N(0, I/d) plus a +0.25 shift on 16 seeded coordinates, Exp(1)-normalised
  weights, eps annealed 1.0 -> 0.01 over 10 stages x 20 iterations, then
  U = P.V with V ~ N(0, I) of width 1024.
* ``c5`` 250k x 250k points in 3-D, X uniform in the unit cube, Y an
  8-component Gaussian mixture (means uniform in the cube, std 0.05),
  uniform weights, eps 0.01, 10 iterations.
* ``fs2`` (the block-sparse form) 250k x 250k points, two independent
  uniform samples of the unit cube, eps = n^(-2/3) (entropic blur equal to
  the mean interparticle distance), annealed from 0.1 over 12 stages.

Every recipe accepts smaller ``n``/``m`` (and, where it makes sense, ``d``)
so the same distributions can be drawn at sizes the oracle finishes in
seconds.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "make", "CONFIGS", "random_cloud"]


@dataclasses.dataclass
class Workload:
    """One synthetic problem instance (all arrays float32, C-contiguous)."""

    name: str
    X: np.ndarray  # (n, d)
    Y: np.ndarray  # (m, d)
    a: np.ndarray  # (n,)
    b: np.ndarray  # (m,)
    eps: float  # regularisation of a single-stage run (final eps if annealed)
    iters: int  # iterations per stage
    n_stages: int = 1
    eps_start: Optional[float] = None  # annealed runs: first-stage eps
    V: Optional[np.ndarray] = None  # (m, dv) right-hand side of P.V, if any
    divide_by_a: bool = False  # True: barycentric projection P.V / a
    seed: int = 0

    @property
    def n(self) -> int:
        return int(self.X.shape[0])

    @property
    def m(self) -> int:
        return int(self.Y.shape[0])

    @property
    def d(self) -> int:
        return int(self.X.shape[1])

    @property
    def total_iters(self) -> int:
        return self.iters * self.n_stages


def _f32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))


def _uniform_weights(k: int) -> np.ndarray:
    return _f32(np.full(k, 1.0 / k))


def _exp_weights(rng: np.random.Generator, k: int) -> np.ndarray:
    # Dirichlet(1,...,1) is i.i.d. Exp(1) normalised; normalised in float64.
    e = rng.standard_exponential(k)
    return _f32(e / e.sum())


def _c1(seed, n=512, m=512, d=3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d)) + 0.5
    return Workload("c1", _f32(X), _f32(Y), _uniform_weights(n), _uniform_weights(m),
                    eps=0.1, iters=100, seed=seed)


def _c2(seed, n=10_000, m=10_000, d=64):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d)) / np.sqrt(d)
    mu = rng.standard_normal(d) / np.sqrt(d)
    Y = mu + np.sqrt(0.5 / d) * rng.standard_normal((m, d))
    return Workload("c2", _f32(X), _f32(Y), _uniform_weights(n), _uniform_weights(m),
                    eps=0.05, iters=200, seed=seed)


def _mixture(rng, k, count, d, std):
    means = rng.standard_normal((k, d)) / np.sqrt(d)
    comp = rng.integers(0, k, size=count)
    return means[comp] + std * rng.standard_normal((count, d))


def _c3(seed, n=50_000, m=50_000, d=512):
    rng = np.random.default_rng(seed)
    std = 0.3 / np.sqrt(d)
    X = _mixture(rng, 10, n, d, std)
    Y = _mixture(rng, 10, m, d, std)
    a = _exp_weights(rng, n)
    b = _exp_weights(rng, m)
    Yf = _f32(Y)
    return Workload("c3", _f32(X), Yf, a, b, eps=0.1, iters=100, V=Yf,
                    divide_by_a=True, seed=seed)


def _c4(seed, n=50_000, m=30_000, d=1024, dv=None):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((n, d))
    X = Z / np.linalg.norm(Z, axis=1, keepdims=True)
    del Z
    Y = rng.standard_normal((m, d)) / np.sqrt(d)
    shift_coords = rng.choice(d, size=min(16, d), replace=False)
    Y[:, shift_coords] += 0.25
    a = _exp_weights(rng, n)
    b = _exp_weights(rng, m)
    V = rng.standard_normal((m, d if dv is None else dv))
    return Workload("c4", _f32(X), _f32(Y), a, b, eps=0.01, iters=20, n_stages=10,
                    eps_start=1.0, V=_f32(V), divide_by_a=False, seed=seed)


def _c5(seed, n=250_000, m=250_000, d=3):
    rng = np.random.default_rng(seed)
    X = rng.random((n, d))
    means = rng.random((8, d))
    comp = rng.integers(0, 8, size=m)
    Y = means[comp] + 0.05 * rng.standard_normal((m, d))
    return Workload("c5", _f32(X), _f32(Y), _uniform_weights(n), _uniform_weights(m),
                    eps=0.01, iters=10, seed=seed)


def _fs2(seed, n=250_000, m=250_000, d=3):
    # Two independent uniform samples of the unit cube at eps = (mean spacing)^2
    # = n^(-2/3): the regime of the block-sparse form (entropic blur equal to
    # the interparticle distance, as in the "FlashSinkhorn 2" explainer's
    # large experiment), annealed from 0.1 over 12 stages of 10 iterations.
    rng = np.random.default_rng(seed)
    X = rng.random((n, d))
    Y = rng.random((m, d))
    return Workload("fs2", _f32(X), _f32(Y), _uniform_weights(n), _uniform_weights(m),
                    eps=float(n) ** (-2.0 / d), iters=10, n_stages=12, eps_start=0.1, seed=seed)


_BUILDERS = {"c1": _c1, "c2": _c2, "c3": _c3, "c4": _c4, "c5": _c5, "fs2": _fs2}

#: full-size shapes of the five recipes, (n, m, d)
CONFIGS = {
    "c1": (512, 512, 3),
    "c2": (10_000, 10_000, 64),
    "c3": (50_000, 50_000, 512),
    "c4": (50_000, 30_000, 1024),
    "c5": (250_000, 250_000, 3),
}

#: the block-sparse form's workload (not one of the five recipes above)
FS2_CONFIG = (250_000, 250_000, 3)

_DEFAULT_SEED = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "fs2": 6}


def make(name: str, n: Optional[int] = None, m: Optional[int] = None,
         d: Optional[int] = None, seed: Optional[int] = None, **kw) -> Workload:
    """Draw recipe ``name`` (``c1`` .. ``c5``, ``fs2``), optionally at a smaller size."""
    name = name.lower()
    if name not in _BUILDERS:
        raise KeyError(f"unknown workload {name!r}; choose from {sorted(_BUILDERS)}")
    n0, m0, d0 = FS2_CONFIG if name == "fs2" else CONFIGS[name]
    s = _DEFAULT_SEED[name] if seed is None else int(seed)
    return _BUILDERS[name](s, n=n or n0, m=m or m0, d=d or d0, **kw)


def random_cloud(seed: int, n: int, m: int, d: int, *, offset: float = 0.5,
                 scale: float = 1.0, weights: str = "uniform", dv: int = 0) -> Workload:
    """A generic Gaussian pair (X ~ N(0, s^2 I), Y ~ N(offset, s^2 I)).

    ``weights`` is ``"uniform"`` or ``"exp"`` (normalised Exp(1)).  ``dv > 0``
    also draws a right-hand side V ~ N(0, I) of width ``dv``.
    """
    rng = np.random.default_rng(seed)
    X = scale * rng.standard_normal((n, d))
    Y = scale * rng.standard_normal((m, d)) + offset
    if weights == "uniform":
        a, b = _uniform_weights(n), _uniform_weights(m)
    elif weights == "exp":
        a, b = _exp_weights(rng, n), _exp_weights(rng, m)
    else:
        raise ValueError(weights)
    V = _f32(rng.standard_normal((m, dv))) if dv > 0 else None
    return Workload("random", _f32(X), _f32(Y), a, b, eps=0.1, iters=10, V=V, seed=seed)
