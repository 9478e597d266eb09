"""float64 CPU oracle of the log-domain Sinkhorn iteration (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; the product path never imports
it.  The arithmetic lives in ``oracle.c`` (see its header for the formulas and
their source on the pages); this module only widens float32 inputs to float64
exactly, calls the C functions and returns numpy arrays.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, a dense scaling-form Sinkhorn, brute-force assignment,
1-D sorted matching and exact metamorphic relations; the gradient and the
dual objective by central finite differences of the converged dual value,
by translation invariance and by the single-target closed form
(``tests/test_oracle_gradient.py``).  ``oracle/hvp.py`` (numpy, dense) holds
the Hessian-vector product, pinned by finite differences of the gradient at
re-converged potentials, symmetry and a closed form
(``tests/test_oracle_hvp.py``).  ``oracle/blocksparse.py`` (numpy) holds the
block-sparse form (Morton order, block bounds, screening, retained-block
update; ``tests/test_oracle_blocksparse.py``) and ``oracle/coarse.py`` its
coarse stage (centroids, lift, sampled marginal check;
``tests/test_oracle_coarse.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_I32 = ctypes.POINTER(ctypes.c_int32)


def compile_library(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (see oracle/build.py)."""
    from .build import build as _build

    return _build(force=force)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    compile_library(force=False)  # no-op unless missing or older than oracle.c
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_version.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_f_update.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_double, _D]
    lib.oracle_g_update.argtypes = lib.oracle_f_update.argtypes
    lib.oracle_f_update_rows.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_double, _I64, ctypes.c_int64, _D]
    lib.oracle_g_update_cols.argtypes = lib.oracle_f_update_rows.argtypes
    lib.oracle_marginal_residual.restype = ctypes.c_double
    lib.oracle_marginal_residual.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_double, _D, _D]
    lib.oracle_stage_eps.restype = ctypes.c_double
    lib.oracle_stage_eps.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                     ctypes.c_double]
    lib.oracle_sinkhorn.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_int32, ctypes.c_double,
                                    ctypes.c_int32, _D, _D, _D, _D, _I32]
    lib.oracle_transport.argtypes = [_D, _D, _D, _D, _D, _D, _D, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_double, ctypes.c_int32, _I64,
                                     ctypes.c_int64, _D]
    lib.oracle_gradient.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_double, _D, _D]
    lib.oracle_dual_objective.restype = ctypes.c_double
    lib.oracle_dual_objective.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
    for name in ("oracle_f_update", "oracle_g_update", "oracle_f_update_rows",
                 "oracle_g_update_cols", "oracle_sinkhorn", "oracle_transport",
                 "oracle_gradient"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    # float32 -> float64 widening is exact.
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x: np.ndarray):
    return x.ctypes.data_as(_D)


def _check(rc: int):
    if rc != 0:
        raise MemoryError("oracle: allocation failed")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def version() -> int:
    return int(_load().oracle_version())


def f_update(X, Y, b, g, eps: float) -> np.ndarray:
    """f_i = -eps LSE_j[(g_j - |x_i - y_j|^2)/eps + log b_j] for every row."""
    lib = _load()
    X, Y, b, g = _f64(X), _f64(Y), _f64(b), _f64(g)
    n, d = X.shape
    m = Y.shape[0]
    out = np.empty(n)
    _check(lib.oracle_f_update(_p(X), _p(Y), _p(b), _p(g), n, m, d, float(eps), _p(out)))
    return out


def g_update(X, Y, a, f, eps: float) -> np.ndarray:
    """g_j = -eps LSE_i[(f_i - |x_i - y_j|^2)/eps + log a_i] for every column."""
    lib = _load()
    X, Y, a, f = _f64(X), _f64(Y), _f64(a), _f64(f)
    n, d = X.shape
    m = Y.shape[0]
    out = np.empty(m)
    _check(lib.oracle_g_update(_p(X), _p(Y), _p(a), _p(f), n, m, d, float(eps), _p(out)))
    return out


def f_update_rows(X, Y, b, g, eps: float, rows: Sequence[int]) -> np.ndarray:
    """The f-update evaluated at the listed rows only."""
    lib = _load()
    X, Y, b, g = _f64(X), _f64(Y), _f64(b), _f64(g)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    m, d = Y.shape
    out = np.empty(rows.shape[0])
    _check(lib.oracle_f_update_rows(_p(X), _p(Y), _p(b), _p(g), m, d, float(eps),
                                    rows.ctypes.data_as(_I64), rows.shape[0], _p(out)))
    return out


def g_update_cols(X, Y, a, f, eps: float, cols: Sequence[int]) -> np.ndarray:
    """The g-update evaluated at the listed columns only."""
    lib = _load()
    X, Y, a, f = _f64(X), _f64(Y), _f64(a), _f64(f)
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    n, d = X.shape
    out = np.empty(cols.shape[0])
    _check(lib.oracle_g_update_cols(_p(X), _p(Y), _p(a), _p(f), n, d, float(eps),
                                    cols.ctypes.data_as(_I64), cols.shape[0], _p(out)))
    return out


def stage_eps(s: int, n_stages: int, eps0: float, eps_end: float) -> float:
    return float(_load().oracle_stage_eps(s, n_stages, eps0, eps_end))


def sinkhorn(X, Y, a, b, *, eps: float, iters: int, n_stages: int = 1,
             eps_start: Optional[float] = None, tol: float = 0.0, check_every: int = 10,
             g0=None, log_dual: bool = False):
    """Alternating log-domain Sinkhorn.  Returns a dict with f, g, iters,
    residual (or -1 when never evaluated) and, if asked, the dual log."""
    lib = _load()
    X, Y, a, b = _f64(X), _f64(Y), _f64(a), _f64(b)
    n, d = X.shape
    m = Y.shape[0]
    f = np.zeros(n)
    g = np.zeros(m) if g0 is None else _f64(g0).copy()
    total = iters * n_stages
    dual = np.full(2 * total, np.nan) if log_dual else None
    resid = ctypes.c_double(-1.0)
    done = ctypes.c_int32(0)
    e0 = eps if eps_start is None else eps_start
    _check(lib.oracle_sinkhorn(_p(X), _p(Y), _p(a), _p(b), n, m, d, n_stages, float(e0),
                               float(eps), iters, float(tol), check_every, _p(f), _p(g),
                               _p(dual) if dual is not None else None,
                               ctypes.byref(resid), ctypes.byref(done)))
    out = {"f": f, "g": g, "iters": int(done.value), "residual": float(resid.value)}
    if dual is not None:
        out["dual"] = dual[: 2 * done.value]
    return out


def marginal_residual(X, Y, a, b, f, g, eps: float):
    """(total, row term, column term) of the L1 marginal residual."""
    lib = _load()
    X, Y, a, b, f, g = (_f64(v) for v in (X, Y, a, b, f, g))
    n, d = X.shape
    m = Y.shape[0]
    r1, r2 = ctypes.c_double(), ctypes.c_double()
    tot = lib.oracle_marginal_residual(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), n, m, d,
                                       float(eps), ctypes.byref(r1), ctypes.byref(r2))
    return float(tot), float(r1.value), float(r2.value)


def transport_t(X, Y, a, b, f, g, W, eps: float, divide_by_b: bool = False,
                cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """U_j = sum_i P_ij W_i (or / b_j): the plan of the swapped problem
    (Y, X, b, a, g, f) is P transposed, so this is `transport` of that
    problem."""
    return transport(Y, X, b, a, g, f, W, eps, divide_by_a=divide_by_b, rows=cols)


def gradient(X, Y, a, b, f, g, eps: float):
    """(grad_x, grad_y) of the dual objective at fixed (f, g):
    grad_x_i = 2 sum_j P_ij (x_i - y_j), grad_y_j = 2 sum_i P_ij (y_j - x_i)."""
    lib = _load()
    X, Y, a, b, f, g = (_f64(v) for v in (X, Y, a, b, f, g))
    n, d = X.shape
    m = Y.shape[0]
    gX = np.empty((n, d))
    gY = np.empty((m, d))
    _check(lib.oracle_gradient(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), n, m, d, float(eps),
                               _p(gX), _p(gY)))
    return gX, gY


def dual_objective(X, Y, a, b, f, g, eps: float) -> float:
    """D = <a,f> + <b,g> - eps sum_ij a_i b_j (exp((f_i + g_j - C_ij)/eps) - 1)."""
    lib = _load()
    X, Y, a, b, f, g = (_f64(v) for v in (X, Y, a, b, f, g))
    n, d = X.shape
    m = Y.shape[0]
    return float(lib.oracle_dual_objective(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), n, m, d,
                                           float(eps)))


def transport(X, Y, a, b, f, g, V, eps: float, divide_by_a: bool = False,
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """U = P.V (or P.V / a), optionally for a subset of rows."""
    lib = _load()
    X, Y, a, b, f, g, V = (_f64(v) for v in (X, Y, a, b, f, g, V))
    n, d = X.shape
    m = Y.shape[0]
    dv = V.shape[1]
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        cnt = rows.shape[0]
        rp = rows.ctypes.data_as(_I64)
    else:
        cnt, rp = n, None
    U = np.empty((cnt, dv))
    _check(lib.oracle_transport(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), _p(V), n, m, d,
                                dv, float(eps), int(bool(divide_by_a)), rp, cnt, _p(U)))
    return U
