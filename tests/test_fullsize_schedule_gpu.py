"""Full-size, full-schedule parity: each recipe at its real shape, in the
precision and launch configuration bench.py times (the same calls on the
same sizes: fs_potentials_init with the recipe's transport width, one
fs_sinkhorn_solve over the whole schedule from g = 0, then the transport),
compared element by element with the float64 oracle after the same
iterations.

Expected values: tests/golden/<recipe>_oracle_full.npz, written by
tests/golden/make_golden_full.py from oracle/ alone (the 50k recipes with
the matrix-product form of the same update, cross-checked there against the
direct-difference oracle).  The streamed update is the exact log-domain
update ("FlashSinkhorn" explainer, "Method" part 2: online LSE, no
approximation), so the iterates are compared one for one.

Bars (every potential, every entry):
  max |f - f_ref|, max |g - g_ref| <= 1e-3 eps   fp32 score paths (c2, c5)
                                   <= 2e-2 eps   bf16 / fp16 paths (c3, c4)
  transport (P.Y / a for c3, P.V for c4) on the oracle's 512 seeded rows:
      ||U - U_ref||_F / ||U_ref||_F <= 1e-3.
The c2 recipe also reports the L1 marginal residual; it is compared with the
oracle's within 2e-2 of its value, plus 4e-6 for the fp32 evaluation floor
(about 1e-6 |f| / eps per term, with |f| ~ 0.2 here).
"""
import json
import os

import numpy as np
import pytest

from helpers import dev, host
from streaming_sinkhorn_solver_amd import workloads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# recipe -> (score precision, expected path, potential bar in eps, fp16
# iterations of a refined solve: the 1024-D recipe runs its whole last stage
# on the fp16 copies, as bench.py does)
RECIPES = {
    "c2": ("fp32", "fp32-mfma", 1e-3, 0),
    "c3": ("bf16-refine", "bf16-mfma-fp16-refine", 2e-2, 0),
    "c3-fp16": ("fp16", "fp16-mfma", 2e-2, 0),
    "c4": ("bf16-refine", "bf16-mfma-fp16-refine", 2e-2, 20),
    "c4-fp16": ("fp16", "fp16-mfma", 2e-2, 0),
    "c5": ("auto", "fp32-small-mfma", 1e-3, 0),
}


def _golden(name):
    path = os.path.join(GOLDEN, f"{name}_oracle_full.npz")
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} has not been written "
                    "(python tests/golden/make_golden_full.py)")
    with open(os.path.join(GOLDEN, f"{name}_oracle_full.json")) as fh:
        meta = json.load(fh)
    with np.load(path, allow_pickle=False) as z:
        return {k: z[k] for k in z.files}, meta


@pytest.mark.parametrize("name", sorted(RECIPES))
def test_full_schedule_against_oracle(fs, name):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    prec, path, bar, refine = RECIPES[name]
    name = name.split("-")[0]
    ref, meta = _golden(name)
    w = workloads.make(name)
    assert (meta["n"], meta["m"], meta["d"], meta["iterations"]) == \
        (w.n, w.m, w.d, w.iters * w.n_stages)
    print(f"{name}: {w.n} x {w.m} x {w.d}, {prec}, {w.iters * w.n_stages} iterations",
          flush=True)
    X, Y, a, b = dev(w.X), dev(w.Y), dev(w.a), dev(w.b)
    V = dev(w.V) if w.V is not None else None
    dv = 0 if V is None else V.shape[1]
    f = torch.empty(w.n, device="cuda")
    g = torch.empty(w.m, device="cuda")
    ws = torch.empty(binding.fs_workspace_bytes(w.n, w.m, w.d, dv, prec) + 256,
                     dtype=torch.uint8, device="cuda")
    p = binding.fs_potentials_init(X, Y, a, b, dv_max=dv, prec=prec, f=f, g=g, workspace=ws)
    assert p.info["path"] == path
    info = binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, eps_start=w.eps_start,
                                     n_stages=w.n_stages, iters_per_stage=w.iters,
                                     refine_iters=refine)
    assert info["iters_done"] == w.iters * w.n_stages
    U = None
    if dv:
        U = torch.empty((w.n, dv), device="cuda")
        binding.fs_apply_transport(p, w.eps, f, g, V, U, divide_by_a=w.divide_by_a)
    torch.cuda.synchronize()
    fh, gh = host(f), host(g)
    ef = float(np.max(np.abs(fh - ref["f"]))) / w.eps
    eg = float(np.max(np.abs(gh - ref["g"]))) / w.eps
    msg = (f"{name}: max|f - f_ref| = {ef:.3e} eps, max|g - g_ref| = {eg:.3e} eps "
           f"(bar {bar:g}); splits {p.info['f_splits']}/{p.info['g_splits']}")
    if U is not None:
        rows = ref["rows"]
        got = host(U)[rows]
        rel = float(np.linalg.norm(got - ref["U_rows"]) / np.linalg.norm(ref["U_rows"]))
        worst = float(np.max(np.linalg.norm(got - ref["U_rows"], axis=1) /
                             np.linalg.norm(ref["U_rows"], axis=1)))
        msg += f"; transport rel {rel:.3e} (worst row {worst:.3e}) on {len(rows)} rows"
    if "residual" in ref:
        out2 = torch.empty(2, device="cuda")
        binding.fs_marginal_residual(p, w.eps, f, g, out2)
        r_gpu = float(host(out2).sum())
        r_ref = float(ref["residual"][0])
        msg += f"; residual {r_gpu:.4e} vs oracle {r_ref:.4e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(fh)) and np.all(np.isfinite(gh))
    assert ef <= bar and eg <= bar
    if U is not None:
        assert rel <= 1e-3
    if "residual" in ref:
        assert abs(r_gpu - r_ref) <= 2e-2 * r_ref + 4e-6


def test_c3_bf16_potentials(fs):
    """The 50k x 50k x 512 recipe in bf16 over its 100 iterations: potentials
    within the 2e-2 eps bar of the oracle (measured 3.2e-3 eps)."""
    ref, _ = _golden("c3")
    f, g, _ = _run_c3_bf16()
    w = workloads.make("c3")
    ef = float(np.max(np.abs(f - ref["f"]))) / w.eps
    eg = float(np.max(np.abs(g - ref["g"]))) / w.eps
    print(f"c3 bf16: max|f - f_ref| = {ef:.3e} eps, max|g - g_ref| = {eg:.3e} eps")
    assert ef <= 2e-2 and eg <= 2e-2


@pytest.mark.xfail(strict=True, reason=(
    "bf16 operands keep 8 significant bits: after the 100 iterations of the 50k x 50k x "
    "512 recipe the potentials sit about 3e-3 eps from the float64 iteration, which moves "
    "the barycentric projection P.Y/a by about 1.2e-3 relative (Frobenius over the 512 "
    "stored rows), just over the 1e-3 bar; the recipe runs with its last iteration and "
    "the projection on fp16 copies (FS_PREC_BF16_REFINE: 1.6e-4 measured)"))
def test_c3_bf16_transport(fs):
    ref, _ = _golden("c3")
    _, _, U = _run_c3_bf16()
    rows = ref["rows"]
    rel = float(np.linalg.norm(U[rows] - ref["U_rows"]) / np.linalg.norm(ref["U_rows"]))
    print(f"c3 bf16 transport rel {rel:.3e}")
    assert rel <= 1e-3


_C3_BF16 = {}


def _run_c3_bf16():
    import torch

    from streaming_sinkhorn_solver_amd import binding

    if "out" not in _C3_BF16:
        w = workloads.make("c3")
        X, Y, a, b, V = dev(w.X), dev(w.Y), dev(w.a), dev(w.b), dev(w.V)
        f = torch.empty(w.n, device="cuda")
        g = torch.empty(w.m, device="cuda")
        p = binding.fs_potentials_init(X, Y, a, b, dv_max=w.d, prec="bf16", f=f, g=g)
        binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=w.iters)
        U = torch.empty((w.n, w.d), device="cuda")
        binding.fs_apply_transport(p, w.eps, f, g, V, U, divide_by_a=True)
        torch.cuda.synchronize()
        _C3_BF16["out"] = (host(f), host(g), host(U))
    return _C3_BF16["out"]
