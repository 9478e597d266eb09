"""Thin ctypes binding of ``libfs_sinkhorn.so`` (the C ABI in include/fs_sinkhorn.h
and include/fs_probe.h).

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the solver runs in the library's kernels.  If the
library has not been built the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "FS_OK", "FS_ERR_INVALID_ARG", "FS_ERR_WORKSPACE", "FS_ERR_DEVICE", "FS_ERR_NONFINITE",
    "FS_ERR_NOT_CONVERGED", "PREC_AUTO", "PREC_FP32", "PREC_BF16", "PREC_FP16", "PREC_FP32_VALU",
    "PREC_BF16_REFINE",
    "FsError",
    "Problem", "load", "lib_path", "fs_workspace_bytes", "fs_potentials_init",
    "fs_lse_update_f", "fs_lse_update_g", "fs_marginal_residual", "fs_sinkhorn_solve",
    "fs_apply_transport", "fs_problem_info", "fs_status_string", "fs_last_error", "solve",
    "PROBE_KINDS", "fs_probe_peak", "fs_apply_transport_t", "fs_gradient", "fs_dual_value",
    "fs_hvp", "fs_hvp_workspace_bytes",
    "COST_SQEUCLIDEAN", "COST_COSINE",
    "fs_morton_workspace_bytes", "fs_morton_sort", "fs_unpermute", "fs_bs_workspace_bytes",
    "fs_bs_attach", "fs_bs_lse_update_f", "fs_bs_lse_update_g", "fs_bs_sinkhorn_solve",
    "fs_bs_shape", "fs_bs_read_screen", "fs_centroids", "fs_lift",
    "fs_sampled_marginal_error", "fs_bs_coarse_start", "fs_bs_apply_transport",
    "fs_bs_apply_transport_t", "fs_bs_gradient", "fs_static_scratch_bytes",
    "fs_sinkhorn_solve_static",
]

FS_OK, FS_ERR_INVALID_ARG, FS_ERR_WORKSPACE, FS_ERR_DEVICE, FS_ERR_NONFINITE, \
    FS_ERR_NOT_CONVERGED = range(6)
PREC_AUTO, PREC_FP32, PREC_BF16, PREC_FP16, PREC_FP32_VALU, PREC_BF16_REFINE = range(6)
_PREC_NAMES = {"auto": PREC_AUTO, "fp32": PREC_FP32, "bf16": PREC_BF16, "fp16": PREC_FP16,
               "fp32-valu": PREC_FP32_VALU, "bf16-refine": PREC_BF16_REFINE}
COST_SQEUCLIDEAN, COST_COSINE = 0, 1
_COST_NAMES = {"sqeuclidean": COST_SQEUCLIDEAN, "cosine": COST_COSINE}
PROBE_KINDS = {"mfma-bf16": 1, "mfma-fp16": 2, "mfma-fp32": 3, "exp": 4}
PATH_NAMES = {0: "fp32-valu", 1: "fp32-mfma", 2: "bf16-mfma", 3: "fp16-mfma", 4: "fp32-small-mfma",
              5: "bf16-mfma-fp16-refine"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.environ.get("FS_SINKHORN_LIB") or os.path.join(_HERE, "libfs_sinkhorn.so")


class SolveOpts(ctypes.Structure):
    _fields_ = [("n_stages", ctypes.c_int32), ("eps_start", ctypes.c_float),
                ("eps_end", ctypes.c_float), ("iters_per_stage", ctypes.c_int32),
                ("tol", ctypes.c_float), ("check_every", ctypes.c_int32),
                ("warm_start", ctypes.c_int32), ("time_kernels", ctypes.c_int32),
                ("single_launch", ctypes.c_int32), ("refine_iters", ctypes.c_int32)]


class SolveInfo(ctypes.Structure):
    _fields_ = [("iters_done", ctypes.c_int32), ("final_eps", ctypes.c_float),
                ("residual", ctypes.c_float), ("lse_launches", ctypes.c_int32),
                ("lse_ms", ctypes.c_float), ("single_launch", ctypes.c_int32)]


class HvpInfo(ctypes.Structure):
    _fields_ = [("cg_iters", ctypes.c_int32), ("cg_residual", ctypes.c_float)]


class CoarseInfo(ctypes.Structure):
    _fields_ = [("rounds", ctypes.c_int32), ("accepted", ctypes.c_int32),
                ("err_rows", ctypes.c_float), ("err_cols", ctypes.c_float)]


class FsError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {message}")


def _status_name(s: int) -> str:
    lib = _LIB
    if lib is None:
        return str(s)
    return lib.fs_status_string(s).decode()


_vp = ctypes.c_void_p
_fp = ctypes.c_void_p  # device float* passed as an address


def load():
    """Load the HIP library (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    i64, i32, f32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.fs_workspace_bytes.restype = sz
    lib.fs_workspace_bytes.argtypes = [i64, i64, i32, i32, ctypes.c_int]
    lib.fs_potentials_init.restype = ctypes.c_int
    lib.fs_potentials_init.argtypes = [_fp, _fp, _fp, _fp, i64, i64, i32, i32, ctypes.c_int,
                                       _vp, sz, _fp, _fp, _vp, ctypes.POINTER(_vp)]
    lib.fs_lse_update_f.restype = ctypes.c_int
    lib.fs_lse_update_f.argtypes = [_vp, f32, _fp, _fp, _fp, _fp, _vp]
    lib.fs_lse_update_g.restype = ctypes.c_int
    lib.fs_lse_update_g.argtypes = [_vp, f32, _fp, _fp, _fp, _fp, _vp]
    lib.fs_marginal_residual.restype = ctypes.c_int
    lib.fs_marginal_residual.argtypes = [_vp, f32, _fp, _fp, _fp, _vp]
    lib.fs_sinkhorn_solve.restype = ctypes.c_int
    lib.fs_sinkhorn_solve.argtypes = [_vp, ctypes.POINTER(SolveOpts), _fp, _fp,
                                      ctypes.POINTER(SolveInfo), _vp]
    lib.fs_apply_transport.restype = ctypes.c_int
    lib.fs_apply_transport.argtypes = [_vp, f32, _fp, _fp, _fp, i32, _fp, i32, _vp]
    lib.fs_destroy.restype = None
    lib.fs_destroy.argtypes = [_vp]
    lib.fs_status_string.restype = ctypes.c_char_p
    lib.fs_status_string.argtypes = [ctypes.c_int]
    lib.fs_last_error.restype = ctypes.c_char_p
    lib.fs_last_error.argtypes = []
    lib.fs_problem_info.restype = ctypes.c_int
    lib.fs_problem_info.argtypes = [_vp] + [ctypes.POINTER(i32)] * 4
    lib.fs_potentials_init_cost.restype = ctypes.c_int
    lib.fs_potentials_init_cost.argtypes = [_fp, _fp, _fp, _fp, i64, i64, i32, i32,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, sz,
                                            _fp, _fp, _vp, ctypes.POINTER(_vp)]
    lib.fs_apply_transport_t.restype = ctypes.c_int
    lib.fs_apply_transport_t.argtypes = [_vp, f32, _fp, _fp, _fp, i32, _fp, i32, _vp]
    lib.fs_gradient.restype = ctypes.c_int
    lib.fs_gradient.argtypes = [_vp, f32, _fp, _fp, _fp, _fp, _fp, _fp, _vp]
    lib.fs_dual_value.restype = ctypes.c_int
    lib.fs_dual_value.argtypes = [_vp, _fp, _fp, ctypes.c_void_p, _vp]
    lib.fs_hvp_workspace_bytes.restype = ctypes.c_size_t
    lib.fs_hvp_workspace_bytes.argtypes = [_vp]
    lib.fs_hvp.restype = ctypes.c_int
    lib.fs_hvp.argtypes = [_vp, f32, _fp, _fp, _fp, _fp, i32, _fp, _fp, f32, i32,
                           ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(HvpInfo), _vp]
    lib.fs_probe_peak.restype = ctypes.c_int
    lib.fs_probe_peak.argtypes = [ctypes.c_int, _fp, i32, _vp, ctypes.POINTER(ctypes.c_double)]
    lib.fs_morton_workspace_bytes.restype = sz
    lib.fs_morton_workspace_bytes.argtypes = [i64, i32]
    lib.fs_morton_sort.restype = ctypes.c_int
    lib.fs_morton_sort.argtypes = [_fp, _fp, i64, i32, _fp, _fp, _fp, _vp, sz, _vp]
    lib.fs_unpermute.restype = ctypes.c_int
    lib.fs_unpermute.argtypes = [_fp, _fp, i64, i32, _fp, _vp]
    lib.fs_bs_workspace_bytes.restype = sz
    lib.fs_bs_workspace_bytes.argtypes = [_vp]
    lib.fs_bs_attach.restype = ctypes.c_int
    lib.fs_bs_attach.argtypes = [_vp, _vp, sz, _vp]
    for name in ("fs_bs_lse_update_f", "fs_bs_lse_update_g"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [_vp, f32, f32, _fp, _fp, _fp, _fp, _vp]
    lib.fs_bs_sinkhorn_solve.restype = ctypes.c_int
    lib.fs_bs_sinkhorn_solve.argtypes = [_vp, ctypes.POINTER(SolveOpts), f32, _fp, _fp,
                                         ctypes.POINTER(SolveInfo), _vp]
    lib.fs_bs_shape.restype = ctypes.c_int
    lib.fs_bs_shape.argtypes = [_vp, i32] + [ctypes.POINTER(i32)] * 3
    lib.fs_bs_read_screen.restype = ctypes.c_int
    lib.fs_bs_read_screen.argtypes = [_vp, i32, _vp, _vp, _vp]
    lib.fs_bs_apply_transport.restype = ctypes.c_int
    lib.fs_bs_apply_transport.argtypes = [_vp, f32, f32, _fp, _fp, _fp, i32, _fp, i32, _vp]
    lib.fs_bs_apply_transport_t.restype = ctypes.c_int
    lib.fs_bs_apply_transport_t.argtypes = [_vp, f32, f32, _fp, _fp, _fp, i32, _fp, i32, _vp]
    lib.fs_bs_gradient.restype = ctypes.c_int
    lib.fs_bs_gradient.argtypes = [_vp, f32, f32, _fp, _fp, _fp, _fp, _vp]
    lib.fs_centroids.restype = ctypes.c_int
    lib.fs_centroids.argtypes = [_fp, _fp, i64, i32, i32, _fp, _fp, _vp]
    lib.fs_lift.restype = ctypes.c_int
    lib.fs_lift.argtypes = [_fp, i64, i32, _fp, _vp]
    lib.fs_sampled_workspace_bytes.restype = sz
    lib.fs_sampled_workspace_bytes.argtypes = [i32, i32]
    lib.fs_sampled_marginal_error.restype = ctypes.c_int
    lib.fs_sampled_marginal_error.argtypes = [_fp, _fp, _fp, _fp, i64, i64, i32, f32, _fp, _fp,
                                              _fp, i32, _fp, i32, _fp, _vp, sz, _vp]
    lib.fs_bs_coarse_start.restype = ctypes.c_int
    lib.fs_bs_coarse_start.argtypes = [_vp, ctypes.POINTER(SolveOpts), i32, f32, _fp, _fp, _fp,
                                       _fp,
                                       i64, i64, i32, i32, f32, i32, _fp, i32, _fp, i32, _fp,
                                       _fp, _fp, _fp, _vp, sz, ctypes.POINTER(CoarseInfo), _vp]
    lib.fs_static_scratch_bytes.restype = sz
    lib.fs_static_scratch_bytes.argtypes = []
    lib.fs_sinkhorn_solve_static.restype = ctypes.c_int
    lib.fs_sinkhorn_solve_static.argtypes = [_fp, _fp, _fp, _fp, i64, i64, i32, ctypes.c_int,
                                             ctypes.POINTER(SolveOpts), _fp, _fp,
                                             ctypes.POINTER(SolveInfo), _vp]
    _LIB = lib
    return lib


def fs_status_string(s: int) -> str:
    return load().fs_status_string(int(s)).decode()


def fs_last_error() -> str:
    return load().fs_last_error().decode()


def _check(status: int, where: str, allow=()):
    if status != FS_OK and status not in allow:
        raise FsError(status, where, fs_last_error())
    return status


def _prec(prec) -> int:
    if isinstance(prec, str):
        return _PREC_NAMES[prec.lower()]
    return int(prec)


def _dev(t: Optional[torch.Tensor], name: str, numel: Optional[int] = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements (has {t.numel()})")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class Problem:
    """A problem handle plus the workspace tensor it lives in."""

    def __init__(self, handle, workspace: torch.Tensor, n: int, m: int, d: int, dv_max: int):
        self.handle = handle
        self.workspace = workspace
        self.n, self.m, self.d, self.dv_max = n, m, d, dv_max

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.fs_destroy(self.handle)
            self.handle = None

    @property
    def info(self) -> dict:
        return fs_problem_info(self)


def fs_workspace_bytes(n: int, m: int, d: int, dv_max: int = 0, prec="auto") -> int:
    return int(load().fs_workspace_bytes(n, m, d, dv_max, _prec(prec)))


def fs_potentials_init(X: torch.Tensor, Y: torch.Tensor, a: torch.Tensor, b: torch.Tensor, *,
                       dv_max: int = 0, prec="auto", f: Optional[torch.Tensor] = None,
                       g: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None, cost: str = "sqeuclidean") -> Problem:
    """fs_potentials_init, or fs_potentials_init_cost for cost="cosine"."""
    lib = load()
    n, d = X.shape
    m = Y.shape[0]
    if Y.shape[1] != d:
        raise ValueError("X and Y must have the same number of columns")
    need = lib.fs_workspace_bytes(n, m, d, dv_max, _prec(prec))
    if need == 0:
        _check(FS_ERR_INVALID_ARG, "fs_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=X.device)
    base = workspace.data_ptr()
    aligned = (base + 255) // 256 * 256
    avail = workspace.numel() - (aligned - base)
    h = _vp()
    if cost not in _COST_NAMES:
        raise ValueError(f"cost must be one of {sorted(_COST_NAMES)}")
    if _COST_NAMES[cost] == COST_SQEUCLIDEAN:
        st = lib.fs_potentials_init(_dev(X, "X", n * d), _dev(Y, "Y", m * d), _dev(a, "a", n),
                                    _dev(b, "b", m), n, m, d, dv_max, _prec(prec), aligned,
                                    avail, _dev(f, "f", n), _dev(g, "g", m), _stream(stream),
                                    ctypes.byref(h))
    else:
        st = lib.fs_potentials_init_cost(_dev(X, "X", n * d), _dev(Y, "Y", m * d),
                                         _dev(a, "a", n), _dev(b, "b", m), n, m, d, dv_max,
                                         _prec(prec), _COST_NAMES[cost], aligned, avail,
                                         _dev(f, "f", n), _dev(g, "g", m), _stream(stream),
                                         ctypes.byref(h))
    _check(st, "fs_potentials_init")
    return Problem(h, workspace, n, m, d, dv_max)


def fs_lse_update_f(p: Problem, eps: float, g, f_out, f_cur=None, row_resid=None, stream=None):
    return _check(load().fs_lse_update_f(p.handle, float(eps), _dev(g, "g", p.m),
                                         _dev(f_out, "f_out", p.n), _dev(f_cur, "f_cur", p.n),
                                         _dev(row_resid, "row_resid", 1), _stream(stream)),
                  "fs_lse_update_f")


def fs_lse_update_g(p: Problem, eps: float, f, g_out, g_cur=None, col_resid=None, stream=None):
    return _check(load().fs_lse_update_g(p.handle, float(eps), _dev(f, "f", p.n),
                                         _dev(g_out, "g_out", p.m), _dev(g_cur, "g_cur", p.m),
                                         _dev(col_resid, "col_resid", 1), _stream(stream)),
                  "fs_lse_update_g")


def fs_marginal_residual(p: Problem, eps: float, f, g, out2, stream=None):
    return _check(load().fs_marginal_residual(p.handle, float(eps), _dev(f, "f", p.n),
                                              _dev(g, "g", p.m), _dev(out2, "out2", 2),
                                              _stream(stream)), "fs_marginal_residual")


def fs_sinkhorn_solve(p: Problem, f, g, *, eps_end: float, iters_per_stage: int,
                      n_stages: int = 1, eps_start: Optional[float] = None, tol: float = 0.0,
                      check_every: int = 10, warm_start: bool = False, stream=None,
                      raise_not_converged: bool = True, time_kernels: bool = False,
                      single_launch: int = 0, refine_iters: int = 0) -> dict:
    opts = SolveOpts(int(n_stages), float(eps_start if eps_start is not None else eps_end),
                     float(eps_end), int(iters_per_stage), float(tol), int(check_every),
                     int(bool(warm_start)), int(bool(time_kernels)), int(single_launch),
                     int(refine_iters))
    info = SolveInfo()
    st = load().fs_sinkhorn_solve(p.handle, ctypes.byref(opts), _dev(f, "f", p.n),
                                  _dev(g, "g", p.m), ctypes.byref(info), _stream(stream))
    allow = () if raise_not_converged else (FS_ERR_NOT_CONVERGED,)
    _check(st, "fs_sinkhorn_solve", allow)
    return {"status": st, "iters_done": info.iters_done, "final_eps": info.final_eps,
            "residual": info.residual, "lse_launches": info.lse_launches,
            "lse_ms": info.lse_ms, "single_launch": bool(info.single_launch)}


def fs_apply_transport(p: Problem, eps: float, f, g, V, U, divide_by_a: bool = False,
                       stream=None):
    dv = V.shape[1]
    return _check(load().fs_apply_transport(p.handle, float(eps), _dev(f, "f", p.n),
                                            _dev(g, "g", p.m), _dev(V, "V", p.m * dv), dv,
                                            _dev(U, "U", p.n * dv), int(bool(divide_by_a)),
                                            _stream(stream)), "fs_apply_transport")


def fs_apply_transport_t(p: Problem, eps: float, f, g, W, U, divide_by_b: bool = False,
                         stream=None):
    dv = W.shape[1]
    return _check(load().fs_apply_transport_t(p.handle, float(eps), _dev(f, "f", p.n),
                                              _dev(g, "g", p.m), _dev(W, "W", p.n * dv), dv,
                                              _dev(U, "U", p.m * dv), int(bool(divide_by_b)),
                                              _stream(stream)), "fs_apply_transport_t")


def fs_gradient(p: Problem, eps: float, f, g, X, Y, grad_x=None, grad_y=None, stream=None):
    return _check(load().fs_gradient(p.handle, float(eps), _dev(f, "f", p.n), _dev(g, "g", p.m),
                                     _dev(X, "X", p.n * p.d), _dev(Y, "Y", p.m * p.d),
                                     _dev(grad_x, "grad_x", p.n * p.d),
                                     _dev(grad_y, "grad_y", p.m * p.d), _stream(stream)),
                  "fs_gradient")


def fs_hvp_workspace_bytes(p: Problem) -> int:
    return int(load().fs_hvp_workspace_bytes(p.handle))


def fs_hvp(p: Problem, eps: float, f, g, X, Y, V, HV, cg_tol: float = 1e-4,
           cg_max_iter: int = 200, workspace=None, stream=None, wrt: str = "x") -> dict:
    """Hessian-vector product of the OT loss with respect to X (wrt="x") or
    Y (wrt="y") into HV; returns the CG iterations and final relative
    residual.  `workspace`: a device tensor of at least
    fs_hvp_workspace_bytes(p) bytes (allocated here if None)."""
    if wrt not in ("x", "y"):
        raise ValueError("wrt must be 'x' or 'y'")
    rows = p.n if wrt == "x" else p.m
    need = fs_hvp_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=V.device)
    if not workspace.is_cuda:
        raise TypeError("workspace must be a device tensor")
    info = HvpInfo()
    _check(load().fs_hvp(p.handle, float(eps), _dev(f, "f", p.n), _dev(g, "g", p.m),
                         _dev(X, "X", p.n * p.d), _dev(Y, "Y", p.m * p.d),
                         0 if wrt == "x" else 1, _dev(V, "V", rows * p.d),
                         _dev(HV, "HV", rows * p.d), float(cg_tol),
                         int(cg_max_iter), workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), ctypes.byref(info),
                         _stream(stream)), "fs_hvp")
    return {"cg_iters": info.cg_iters, "cg_residual": info.cg_residual}


def fs_dual_value(p: Problem, f, g, out=None, stream=None) -> torch.Tensor:
    """<a,f> + <b,g> into a one-element float64 device tensor (returned)."""
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=f.device)
    if out.dtype != torch.float64 or not out.is_cuda or out.numel() < 1:
        raise TypeError("out must be a float64 device tensor")
    _check(load().fs_dual_value(p.handle, _dev(f, "f", p.n), _dev(g, "g", p.m), out.data_ptr(),
                                _stream(stream)), "fs_dual_value")
    return out


def fs_problem_info(p: Problem) -> dict:
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(load().fs_problem_info(p.handle, *[ctypes.byref(v) for v in vals]), "fs_problem_info")
    path, dp, fs_, gs = (v.value for v in vals)
    return {"path": PATH_NAMES.get(path, str(path)), "d_pad": dp, "f_splits": fs_,
            "g_splits": gs}


def fs_probe_peak(kind: str, sink, reps: int = 9, stream=None) -> float:
    """Median rate of the unit probe `kind` (a key of PROBE_KINDS): flop/s for
    the matrix-core probes, exponentials/s for "exp".  `sink` is a device
    float tensor of >= 1 element."""
    rate = ctypes.c_double()
    if sink.numel() < 1:
        raise ValueError("sink must have at least one element")
    _check(load().fs_probe_peak(PROBE_KINDS[kind], _dev(sink, "sink"), int(reps),
                                _stream(stream), ctypes.byref(rate)), "fs_probe_peak")
    return rate.value


def _idev(t, name: str, numel: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != numel:
        raise TypeError(f"{name} must be a contiguous int32 tensor of {numel} elements")
    return t.data_ptr()


def fs_morton_workspace_bytes(n: int, d: int) -> int:
    return int(load().fs_morton_workspace_bytes(n, d))


def fs_morton_sort(X, w=None, X_sorted=None, w_sorted=None, perm=None, workspace=None,
                   stream=None):
    """Morton order of the points X (n x d); returns (X_sorted, w_sorted, perm)
    with X_sorted[i] = X[perm[i]] (w_sorted None when w is None)."""
    n, d = X.shape
    dev = X.device
    if X_sorted is None:
        X_sorted = torch.empty_like(X)
    if w is not None and w_sorted is None:
        w_sorted = torch.empty_like(w)
    if perm is None:
        perm = torch.empty(n, dtype=torch.int32, device=dev)
    need = fs_morton_workspace_bytes(n, d)
    if need == 0:
        _check(FS_ERR_INVALID_ARG, "fs_morton_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(load().fs_morton_sort(_dev(X, "X", n * d), _dev(w, "w", n), n, d,
                                 _dev(X_sorted, "X_sorted", n * d), _dev(w_sorted, "w_sorted", n),
                                 _idev(perm, "perm", n), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "fs_morton_sort")
    return X_sorted, w_sorted, perm


def fs_unpermute(src, perm, dst=None, stream=None):
    """dst[perm[i]] = src[i] (rows of src.numel() // n floats)."""
    n = perm.numel()
    width = src.numel() // n
    if dst is None:
        dst = torch.empty_like(src)
    _check(load().fs_unpermute(_dev(src, "src", n * width), _idev(perm, "perm", n), n, width,
                               _dev(dst, "dst", n * width), _stream(stream)), "fs_unpermute")
    return dst


def fs_bs_workspace_bytes(p: Problem) -> int:
    return int(load().fs_bs_workspace_bytes(p.handle))


def fs_bs_attach(p: Problem, workspace=None, stream=None):
    """Enables the block-sparse form; keeps the workspace on the handle."""
    need = fs_bs_workspace_bytes(p)
    if need == 0:
        _check(FS_ERR_INVALID_ARG, "fs_bs_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=p.workspace.device)
    _check(load().fs_bs_attach(p.handle, workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "fs_bs_attach")
    p.bs_workspace = workspace
    return p


def fs_bs_lse_update_f(p: Problem, eps: float, delta: float, g, f_cur, f_out, row_resid=None,
                       stream=None):
    return _check(load().fs_bs_lse_update_f(p.handle, float(eps), float(delta),
                                            _dev(g, "g", p.m), _dev(f_cur, "f_cur", p.n),
                                            _dev(f_out, "f_out", p.n),
                                            _dev(row_resid, "row_resid", 1), _stream(stream)),
                  "fs_bs_lse_update_f")


def fs_bs_lse_update_g(p: Problem, eps: float, delta: float, f, g_cur, g_out, col_resid=None,
                       stream=None):
    return _check(load().fs_bs_lse_update_g(p.handle, float(eps), float(delta),
                                            _dev(f, "f", p.n), _dev(g_cur, "g_cur", p.m),
                                            _dev(g_out, "g_out", p.m),
                                            _dev(col_resid, "col_resid", 1), _stream(stream)),
                  "fs_bs_lse_update_g")


def fs_bs_sinkhorn_solve(p: Problem, f, g, *, eps_end: float, iters_per_stage: int,
                         delta: float, n_stages: int = 1, eps_start: Optional[float] = None,
                         tol: float = 0.0, check_every: int = 10, warm_start: bool = False,
                         stream=None, raise_not_converged: bool = True,
                         time_kernels: bool = False) -> dict:
    opts = SolveOpts(int(n_stages), float(eps_start if eps_start is not None else eps_end),
                     float(eps_end), int(iters_per_stage), float(tol), int(check_every),
                     int(bool(warm_start)), int(bool(time_kernels)))
    info = SolveInfo()
    st = load().fs_bs_sinkhorn_solve(p.handle, ctypes.byref(opts), float(delta),
                                     _dev(f, "f", p.n), _dev(g, "g", p.m), ctypes.byref(info),
                                     _stream(stream))
    allow = () if raise_not_converged else (FS_ERR_NOT_CONVERGED,)
    _check(st, "fs_bs_sinkhorn_solve", allow)
    return {"status": st, "iters_done": info.iters_done, "final_eps": info.final_eps,
            "residual": info.residual, "lse_launches": info.lse_launches,
            "lse_ms": info.lse_ms, "single_launch": bool(info.single_launch)}


def fs_bs_shape(p: Problem, side: int) -> dict:
    vals = [ctypes.c_int32() for _ in range(3)]
    _check(load().fs_bs_shape(p.handle, int(side), *[ctypes.byref(v) for v in vals]),
           "fs_bs_shape")
    return {"row_blocks": vals[0].value, "key_blocks": vals[1].value, "stride": vals[2].value}


def fs_bs_read_screen(p: Problem, side: int, lists: bool = False, stream=None):
    """Kept-block counts per row block of the last screening of `side` (numpy
    int32), and with lists=True the padded lists (row_blocks x stride)."""
    import numpy as np

    sh = fs_bs_shape(p, side)
    counts = np.zeros(sh["row_blocks"], np.int32)
    L = np.zeros((sh["row_blocks"], sh["stride"]), np.int32) if lists else None
    _check(load().fs_bs_read_screen(p.handle, int(side), counts.ctypes.data,
                                    L.ctypes.data if lists else None, _stream(stream)),
           "fs_bs_read_screen")
    return (counts, L) if lists else counts


def fs_bs_apply_transport(p: Problem, eps: float, delta: float, f, g, V, U,
                          divide_by_a: bool = False, stream=None):
    dv = V.shape[1]
    return _check(load().fs_bs_apply_transport(p.handle, float(eps), float(delta),
                                               _dev(f, "f", p.n), _dev(g, "g", p.m),
                                               _dev(V, "V", p.m * dv), dv,
                                               _dev(U, "U", p.n * dv), int(bool(divide_by_a)),
                                               _stream(stream)), "fs_bs_apply_transport")


def fs_bs_apply_transport_t(p: Problem, eps: float, delta: float, f, g, W, U,
                            divide_by_b: bool = False, stream=None):
    dv = W.shape[1]
    return _check(load().fs_bs_apply_transport_t(p.handle, float(eps), float(delta),
                                                 _dev(f, "f", p.n), _dev(g, "g", p.m),
                                                 _dev(W, "W", p.n * dv), dv,
                                                 _dev(U, "U", p.m * dv), int(bool(divide_by_b)),
                                                 _stream(stream)), "fs_bs_apply_transport_t")


def fs_bs_gradient(p: Problem, eps: float, delta: float, f, g, grad_x=None, grad_y=None,
                   stream=None):
    gx = _dev(grad_x, "grad_x", p.n * p.d) if grad_x is not None else None
    gy = _dev(grad_y, "grad_y", p.m * p.d) if grad_y is not None else None
    return _check(load().fs_bs_gradient(p.handle, float(eps), float(delta), _dev(f, "f", p.n),
                                        _dev(g, "g", p.m), gx, gy, _stream(stream)),
                  "fs_bs_gradient")


def fs_centroids(P, w, cell: int, C=None, W=None, stream=None):
    """Centroids and weights of runs of `cell` points; returns (C, W)."""
    n, d = P.shape
    nc = (n + cell - 1) // cell if cell >= 1 else 1  # (the library rejects cell < 1)
    C = torch.empty((nc, d), device=P.device) if C is None else C
    W = torch.empty(nc, device=P.device) if W is None else W
    _check(load().fs_centroids(_dev(P, "P", n * d), _dev(w, "w", n), n, d, int(cell),
                               _dev(C, "C", nc * d), _dev(W, "W", nc), _stream(stream)),
           "fs_centroids")
    return C, W


def fs_lift(F, n: int, cell: int, f=None, stream=None):
    f = torch.empty(n, device=F.device) if f is None else f
    _check(load().fs_lift(_dev(F, "F", (n + cell - 1) // cell), n, int(cell), _dev(f, "f", n),
                          _stream(stream)), "fs_lift")
    return f


def fs_sampled_marginal_error(X, Y, a, b, f, g, eps: float, rows, cols, out2=None,
                              workspace=None, stream=None):
    """(err_rows, err_cols) as a 2-element device tensor."""
    lib = load()
    n, d = X.shape
    m = Y.shape[0]
    nr, nc = rows.numel(), cols.numel()
    out2 = torch.empty(2, device=X.device) if out2 is None else out2
    need = lib.fs_sampled_workspace_bytes(nr, nc)
    workspace = torch.empty(need, dtype=torch.uint8, device=X.device) if workspace is None \
        else workspace
    _check(lib.fs_sampled_marginal_error(
        _dev(X, "X", n * d), _dev(Y, "Y", m * d), _dev(a, "a", n), _dev(b, "b", m), n, m, d,
        float(eps), _dev(f, "f", n), _dev(g, "g", m), _idev(rows, "rows", nr), nr,
        _idev(cols, "cols", nc), nc, _dev(out2, "out2", 2), workspace.data_ptr(),
        workspace.numel(), _stream(stream)), "fs_sampled_marginal_error")
    return out2


def fs_bs_coarse_start(coarse: Problem, X, Y, a, b, cell: int, f, g, F, G, rows, cols, *,
                       eps_end: float, iters_per_stage: int, n_stages: int = 1,
                       eps_start: Optional[float] = None, more_iters: int = 10,
                       check_tol: float = 1e-2, max_rounds: int = 5, coarse_delta: float = 0.0,
                       stream=None) -> dict:
    """The coarse stage (see include/fs_sinkhorn.h); fills F, G (coarse) and
    f, g (lifted); returns rounds, accepted and the last errors.  coarse_delta
    > 0 solves the coarse problem in block-sparse form (attach it first)."""
    lib = load()
    n, d = X.shape
    m = Y.shape[0]
    nr, nc = rows.numel(), cols.numel()
    need = lib.fs_sampled_workspace_bytes(nr, nc) + 256
    ws = torch.empty(need, dtype=torch.uint8, device=X.device)
    opts = SolveOpts(int(n_stages), float(eps_start if eps_start is not None else eps_end),
                     float(eps_end), int(iters_per_stage), 0.0, 1, 0, 0)
    info = CoarseInfo()
    _check(lib.fs_bs_coarse_start(
        coarse.handle, ctypes.byref(opts), int(more_iters), float(coarse_delta),
        _dev(X, "X", n * d),
        _dev(Y, "Y", m * d), _dev(a, "a", n), _dev(b, "b", m), n, m, d, int(cell),
        float(check_tol), int(max_rounds), _idev(rows, "rows", nr), nr, _idev(cols, "cols", nc),
        nc, _dev(F, "F", coarse.n), _dev(G, "G", coarse.m), _dev(f, "f", n), _dev(g, "g", m),
        ws.data_ptr(), need, ctypes.byref(info), _stream(stream)), "fs_bs_coarse_start")
    return {"rounds": info.rounds, "accepted": bool(info.accepted), "err_rows": info.err_rows,
            "err_cols": info.err_cols}


def fs_static_scratch_bytes() -> int:
    return int(load().fs_static_scratch_bytes())


def fs_sinkhorn_solve_static(X, Y, a, b, f, g, *, eps_end: float, iters_per_stage: int,
                             prec="auto", n_stages: int = 1, eps_start: Optional[float] = None,
                             tol: float = 0.0, check_every: int = 10, warm_start: bool = False,
                             stream=None, raise_not_converged: bool = True,
                             refine_iters: int = 0) -> dict:
    """fs_sinkhorn_solve_static: set-up and solve with the library's static
    device scratch as the workspace (no allocation)."""
    n, d = X.shape
    m = Y.shape[0]
    opts = SolveOpts(int(n_stages), float(eps_start if eps_start is not None else eps_end),
                     float(eps_end), int(iters_per_stage), float(tol), int(check_every),
                     int(bool(warm_start)), 0, 0, int(refine_iters))
    info = SolveInfo()
    st = load().fs_sinkhorn_solve_static(_dev(X, "X", n * d), _dev(Y, "Y", m * d),
                                         _dev(a, "a", n), _dev(b, "b", m), n, m, d, _prec(prec),
                                         ctypes.byref(opts), _dev(f, "f", n), _dev(g, "g", m),
                                         ctypes.byref(info), _stream(stream))
    allow = () if raise_not_converged else (FS_ERR_NOT_CONVERGED,)
    _check(st, "fs_sinkhorn_solve_static", allow)
    return {"status": st, "iters_done": info.iters_done, "final_eps": info.final_eps,
            "residual": info.residual}


def solve(X, Y, a, b, *, eps: float, iters: int, prec="auto", n_stages: int = 1,
          eps_start: Optional[float] = None, tol: float = 0.0, check_every: int = 10,
          dv_max: int = 0, cost: str = "sqeuclidean"):
    """Convenience: init + solve; returns (problem, f, g, info)."""
    dev = X.device
    f = torch.empty(X.shape[0], dtype=torch.float32, device=dev)
    g = torch.empty(Y.shape[0], dtype=torch.float32, device=dev)
    p = fs_potentials_init(X, Y, a, b, dv_max=dv_max, prec=prec, f=f, g=g, cost=cost)
    info = fs_sinkhorn_solve(p, f, g, eps_end=eps, iters_per_stage=iters, n_stages=n_stages,
                             eps_start=eps_start, tol=tol, check_every=check_every,
                             raise_not_converged=False)
    return p, f, g, info
