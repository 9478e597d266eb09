#!/usr/bin/env python3
"""Benchmark of the streaming log-sum-exp Sinkhorn solver on one MI355X.

Default workload (the recipe the headline metric is quoted on): n = m =
50,000 points in 512-D, two 10-component Gaussian mixtures, Dirichlet(1)
weights, eps = 0.1, bf16 matrix-core scores with fp32 accumulation.  One step
is the whole hot path on resident inputs: problem preparation (centring,
conversion, per-point cost terms, log-weights), the alternating f/g iterations and the
transport product (here the barycentric projection P.Y / a).

``--workload c1|c2|c4|c5`` runs one of the other recipes the same way (its own
sizes, precision, schedule and transport), for measurements beside the
headline line.  ``--workload fs2`` measures the block-sparse form
(fs_bs_*) on two uniform samples of 250k points in the unit cube at
eps = (mean spacing)^2: the clouds are Morton-ordered and the solve annealed
to the final eps once on the dense path (untimed, reported in `setup`); a step
restores that
warm start and runs 10 block-sparse iterations (fits, screening, the
retained-block LSE passes), `value` being those iterations per second.  Its
`block_sparse` field reports the kept share of block pairs per side, the
dense path's rate on the same potentials and the certificate bound; the c5
line carries the same field for its own clouds and eps.

Prints one JSON line with
  value      Sinkhorn iterations per second over whole steps
  roofline   the streaming LSE kernel (the dominant kernel of every recipe):
             algorithmic work per launch over its mean launch duration, timed
             with HIP events on the launch stream inside the timed region.
             Matrix-core recipes: 2 n m d flops per half-step against the
             MI355X dense peak of the score element type.  d = 3 recipes:
             one exponential per pair against the exponential peak, 256 CUs x
             32 lanes/clock x 2.4 GHz = 19.66e12/s.  `traffic` is the
             per-launch HBM bytes from the committed rocprofv3 counter summary
             when it was taken on the current kernel source, else null.
             `peak_measured` / `frac_measured`: the same against the rate a
             probe kernel of that unit alone (fs_probe_peak: independent chains
             of the score path's matrix instruction, or of v_exp_f32) reaches
             on this GPU right after the timed region
  clocks     mean socket power and graphics clock sampled with amd-smi during
             the timed steps (null when the tool is unavailable).  Context
             only: the tool reports averages over its own window, which for
             runs of a few seconds includes the idle time before them
  phases_ms  mean time per step of problem preparation, the solve and the
             transport (HIP events on the solver's stream)
  transport_roofline  (matrix-core recipes with a transport) the transport
             phase against the same dense peak, counting 2 n m (d + dv)
             flops: the scores and the product with V
  backward   (recipes with a transport of width >= d) one fs_gradient call
             for both clouds at the final potentials, timed after the steps
  cpu_baseline  the float64 oracle's f-update timed on this host's cores on a
             bounded sample of rows of the same workload, scaled to
             iterations per second
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import threading
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "Sinkhorn iters/sec and pair-evals/sec at n=m=50k, d=512; % of roofline"
CSRC = os.path.join(HERE, "streaming_sinkhorn_solver_amd", "csrc")
EXP_PEAK = 256 * 32 * 2.4e9 / 1e12  # T exponentials/s

# recipe -> the fs_probe_peak kind of its bounding unit
PROBES = {"c1": "exp", "c2": "mfma-fp32", "c3": "mfma-bf16", "c4": "mfma-fp16", "c5": "exp",
          "fs2": "exp"}
BS_DELTA = 1e-3  # skipped mass per row / column below this share of its target

# recipe -> (score precision, roofline peak, unit, dtype label, description); the
# d = 3 recipes' label is replaced by what their path takes (small_path_dtype)
# FS_PREC_BF16_REFINE: iterations at the end of the schedule on the fp16
# copies (the 1024-D recipe: its whole last stage; default: the last one)
REFINE_ITERS = {"c4": 20}

RECIPES = {
    "c1": ("auto", EXP_PEAK, "Texp/s", "f32",
           "n=m=512, d=3, X~N(0,I), Y~N(0.5,I), uniform weights, eps=0.1, 100 iterations (seed 1)"),
    "c2": ("fp32", 157.3, "TFLOP/s", "f32",
           "n=m=10000, d=64, X~N(0,I/d), Y~N(mu,0.5 I/d), uniform weights, eps=0.05, "
           "200 iterations (seed 2)"),
    "c3": ("bf16-refine", 2500.0, "TFLOP/s", "bf16 (iterations 1-99); f16 (iteration 100, P.Y/a)",
           "n=m=50000, d=512, two 10-component Gaussian mixtures, Dirichlet(1) weights, "
           "eps=0.1, 100 alternating iterations + barycentric projection P.Y/a (seed 3); "
           "bf16 matrix-core scores with the last iteration and the projection on fp16 "
           "copies of the points (FS_PREC_BF16_REFINE: bf16 throughout misses the 1e-3 "
           "transport bar on this recipe)"),
    "c4": ("bf16-refine", 2500.0, "TFLOP/s", "bf16 (stages 1-9); f16 (stage 10, P.V)",
           "n=50000, m=30000, d=1024, X on the unit sphere, Y~N(0,I/d) with a 0.25 shift on 16 "
           "coordinates, Exp(1) weights, eps 1 -> 0.01 over 10 stages x 20 iterations, "
           "then U=P.V with V~N(0,I), width 1024 (seed 4); bf16 matrix-core scores with the "
           "last stage and the transport on fp16 copies of the points (FS_PREC_BF16_REFINE "
           "with refine_iters = 20: bf16 throughout misses the 2e-2 eps and 1e-3 transport "
           "bars on this recipe)"),
    "c5": ("auto", EXP_PEAK, "Texp/s", "f32",
           "n=m=250000, d=3, X uniform in the unit cube, Y an 8-component mixture (std 0.05), "
           "uniform weights, eps=0.01, 10 iterations (seed 5)"),
    "fs2": ("auto", EXP_PEAK, "Texp/s", "f32",
            "n=m=250000, d=3, two independent uniform samples of the unit cube, uniform "
            "weights, eps=n^(-2/3) (entropic blur = mean spacing), block-sparse form with "
            "delta=1e-3: Morton order, annealed dense warm start 0.1 -> eps over 12 stages x 10 "
            "(untimed), then 10 timed block-sparse iterations per step (seed 6)"),
}


def small_path_dtype(X, Y, a, b, f, g, eps: float) -> str:
    """The score arithmetic the d <= 8 matrix path takes, per half-step: fp16
    hi/lo splits of the products (fp32 accumulation) when its guard holds --
    c_score * max_i sum_c |x'_ic| * max_jc |y'_jc| <= 2^9 on centred points,
    with every magnitude and key bias in the fp16 range -- else bf16
    three-part splits (d <= 4) or fp32 products (d > 4).  Evaluated on the
    host from the inputs and the final potentials, for the label of the
    line."""
    import numpy as np

    log2e = 1.4426950408889634
    c_bias = log2e / eps
    c_score = 2.0 * c_bias
    Xf, Yf = np.asarray(X, np.float32), np.asarray(Y, np.float32)
    nu = ((Xf.min(0) + Xf.max(0)) * np.float32(0.5)).astype(np.float64)
    mu = ((Yf.min(0) + Yf.max(0)) * np.float32(0.5)).astype(np.float64)
    Xc, Yc = Xf.astype(np.float64) - nu, Yf.astype(np.float64) - mu
    h = 0.5 * float((nu - mu) @ (nu - mu))
    A = np.sum((Xf.astype(np.float64) - mu) ** 2, axis=1) - h  # cost term of x
    B = np.sum((Yf.astype(np.float64) - nu) ** 2, axis=1) - h  # cost term of y

    def split_ok(R, K, K_term, K_pot, K_w):
        rl1 = c_score * float(np.max(np.sum(np.abs(R), axis=1)))
        kmax = float(np.max(np.abs(K)))
        beta = (np.asarray(K_pot, np.float64) - K_term) * c_bias + np.log2(np.asarray(K_w, np.float64))
        return (rl1 * kmax <= 512.0 and rl1 <= 16384.0 and kmax <= 16384.0
                and float(np.max(np.abs(beta))) <= 32768.0)

    f_side = split_ok(Xc, Yc, B, g, b)
    g_side = split_ok(Yc, Xc, A, f, a)
    other = "bf16x3-split/f32-acc" if Xf.shape[1] <= 4 else "f32"
    if f_side and g_side:
        return "f16x3-split/f32-acc"
    if not f_side and not g_side:
        return other
    return "f16x3-split/f32-acc (one side), %s (other)" % other


def block_sparse_run(w, eps, steps, warmup, dev, binding, torch):
    """Block-sparse form on the workload's clouds at `eps`: Morton order,
    problem, annealed warm start (0.1 -> eps, 12 x 10, dense path), then
    `steps` timed steps of 10 block-sparse iterations each from that warm
    start; the dense path's 10 iterations from the same start beside it."""
    import numpy as np

    X = torch.from_numpy(w.X).to(dev)
    Y = torch.from_numpy(w.Y).to(dev)
    a = torch.from_numpy(w.a).to(dev)
    b = torch.from_numpy(w.b).to(dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    Xs, a_s, px = binding.fs_morton_sort(X, a)
    Ys, b_s, py = binding.fs_morton_sort(Y, b)
    e[1].record()
    f0 = torch.zeros(w.n, device=dev)
    g0 = torch.zeros(w.m, device=dev)
    p = binding.fs_potentials_init(Xs, Ys, a_s, b_s, f=f0, g=g0, dv_max=w.d)
    binding.fs_bs_attach(p)
    e[2].record()
    # the warm start on the dense path, so that every block-sparse launch of
    # the run is one of the measured configuration (eps, delta)
    binding.fs_sinkhorn_solve(p, f0, g0, eps_end=eps, eps_start=0.1, n_stages=12,
                              iters_per_stage=10)
    e[3].record()
    torch.cuda.synchronize()
    setup = {"morton_sort_ms": round(e[0].elapsed_time(e[1]), 3),
             "init_attach_ms": round(e[1].elapsed_time(e[2]), 3),
             "anneal_ms": round(e[2].elapsed_time(e[3]), 3)}
    f, g = f0.clone(), g0.clone()
    lse = {"ms": 0.0, "n": 0}

    def bs_step(timed):
        f.copy_(f0)
        g.copy_(g0)
        info = binding.fs_bs_sinkhorn_solve(p, f, g, eps_end=eps, iters_per_stage=10,
                                            delta=BS_DELTA, warm_start=True, time_kernels=timed)
        if timed:
            lse["ms"] += info["lse_ms"]
            lse["n"] += info["lse_launches"]

    for _ in range(warmup):
        bs_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        bs_step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kept = {}
    pairs_per_iter = 0.0
    for side, name in ((0, "f"), (1, "g")):
        cnt = binding.fs_bs_read_screen(p, side)
        sh = binding.fs_bs_shape(p, side)
        kept[name] = round(float(cnt.sum()) / (sh["row_blocks"] * sh["key_blocks"]), 5)
        pairs_per_iter += float(cnt.sum()) * 32 * 256  # kept block pairs x pairs per block
    res = torch.zeros(2, device=dev)
    binding.fs_marginal_residual(p, eps, f, g, res)
    # the dense path, same potentials, same iterations
    fd, gd = f0.clone(), g0.clone()
    binding.fs_sinkhorn_solve(p, fd, gd, eps_end=eps, iters_per_stage=10, warm_start=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fd.copy_(f0)
    gd.copy_(g0)
    binding.fs_sinkhorn_solve(p, fd, gd, eps_end=eps, iters_per_stage=10, warm_start=True)
    torch.cuda.synchronize()
    dense_it_s = 10 / (time.perf_counter() - t1)
    it_s = 10 * steps / dt
    # the barycentric projection P.Y / a and the gradient (both clouds) at the
    # final potentials, block-sparse and dense (one untimed call each first)
    U = torch.empty((w.n, w.d), device=dev)
    GX = torch.empty((w.n, w.d), device=dev)
    GY = torch.empty((w.m, w.d), device=dev)
    tr = {}
    for name, call in (("projection_block_sparse", lambda: binding.fs_bs_apply_transport(
            p, eps, BS_DELTA, f, g, Ys, U, divide_by_a=True)),
            ("projection_dense", lambda: binding.fs_apply_transport(
                p, eps, f, g, Ys, U, divide_by_a=True)),
            ("gradient_block_sparse", lambda: binding.fs_bs_gradient(
                p, eps, BS_DELTA, f, g, GX, GY)),
            ("gradient_dense", lambda: binding.fs_gradient(p, eps, f, g, Xs, Ys, GX, GY))):
        call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        tr[name] = round(e0.elapsed_time(e1), 3)
    lse_mean_ms = lse["ms"] / max(lse["n"], 1)
    diff = float((f - fd).abs().max()) / eps
    r = res.cpu().numpy()
    return {
        "iters_per_s": round(it_s, 3), "ms_per_iter": round(dt / (10 * steps) * 1e3, 4),
        "dense_iters_per_s": round(dense_it_s, 3), "speedup_vs_dense": round(it_s / dense_it_s, 3),
        "eps": eps, "delta": BS_DELTA, "kept_block_pairs": kept,
        "kept_pairs_per_iter": pairs_per_iter,
        "lse_mean_launch_ms": round(lse_mean_ms, 4), "lse_launches": lse["n"],
        "dense_marginal_residual_after": [float(r[0]), float(r[1])],
        "max_abs_f_minus_dense_over_eps": round(diff, 4),
        "setup": setup,
        "apply_ms": tr,
        "what": "10 block-sparse iterations from the annealed warm start (per-block fits, "
                "screening, retained-block LSE passes) vs 10 dense iterations from the same "
                "start; kept shares are of the last screening of each side",
    }


def file_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_source_sha(workload: str = "c3") -> str:
    """Hash of the source of the recipe's streaming LSE kernel."""
    return file_sha("fs_lse_small.hip" if workload in ("c1", "c5", "fs2") else "fs_lse.hip")


def traffic_file(workload: str) -> str:
    return os.path.join(HERE, "profiles", f"lse_{workload}_traffic.json")


def counter_mode(w, prec: str, half_steps: int = 6) -> None:
    """Workload for hardware-counter runs: a 1 GiB elementwise read+write of
    known size (the counters' calibration), then problem preparation,
    `half_steps` alternating LSE passes of the recipe at its final eps and,
    for recipes with a transport, one more f-update and two transports."""
    import torch

    from streaming_sinkhorn_solver_amd import binding

    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    X, Y, a, b = (torch.from_numpy(v).to(dev) for v in (w.X, w.Y, w.a, w.b))
    f = torch.empty(w.n, device=dev)
    g = torch.empty(w.m, device=dev)
    if w.name == "fs2":
        # Morton order, a dense annealed warm start (no block-sparse launch
        # before the counted ones), then the block-sparse half-steps
        Xs, a_s, _ = binding.fs_morton_sort(X, a)
        Ys, b_s, _ = binding.fs_morton_sort(Y, b)
        p = binding.fs_potentials_init(Xs, Ys, a_s, b_s, f=f, g=g)
        binding.fs_bs_attach(p)
        binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, eps_start=w.eps_start,
                                  n_stages=w.n_stages, iters_per_stage=w.iters)
        f2, g2 = torch.empty_like(f), torch.empty_like(g)
        for k in range(half_steps):
            if k % 2 == 0:
                binding.fs_bs_lse_update_f(p, w.eps, BS_DELTA, g, f, f2)
                f, f2 = f2, f
            else:
                binding.fs_bs_lse_update_g(p, w.eps, BS_DELTA, f, g, g2)
                g, g2 = g2, g
        torch.cuda.synchronize()
        print(json.dumps({"counter_mode": "done", "half_steps": half_steps,
                          "copy_bytes": float(1 << 30)}), flush=True)
        return
    dv = w.V.shape[1] if w.V is not None else 0
    p = binding.fs_potentials_init(X, Y, a, b, prec=prec, f=f, g=g, dv_max=dv)
    for k in range(half_steps):
        if k % 2 == 0:
            binding.fs_lse_update_f(p, w.eps, g, f)
        else:
            binding.fs_lse_update_g(p, w.eps, f, g)
    transports = 0
    if dv:
        # then the recipe's transport, twice, after one more f-update (so f
        # is its own update's output under g)
        binding.fs_lse_update_f(p, w.eps, g, f)
        V = torch.from_numpy(w.V).to(dev)
        U = torch.empty((w.n, dv), device=dev)
        for _ in range(2):
            binding.fs_apply_transport(p, w.eps, f, g, V, U, divide_by_a=w.divide_by_a)
        transports = 2
    torch.cuda.synchronize()
    print(json.dumps({"counter_mode": "done", "half_steps": half_steps,
                      "transports": transports, "copy_bytes": float(1 << 30)}), flush=True)


def traffic_per_launch(workload: str):
    """Calibrated HBM bytes per LSE launch from the committed counter summary,
    or None if it is missing or was taken on another kernel source."""
    try:
        with open(traffic_file(workload)) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_sha(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


class PowerSampler(threading.Thread):
    """Samples socket power and the graphics clocks with `amd-smi metric`
    while the timed steps run (best effort: no samples if the tool is absent
    or fails)."""

    def __init__(self, gpu: int = 0, period_s: float = 0.5):
        super().__init__(daemon=True)
        self.gpu, self.period = gpu, period_s
        self.halt = threading.Event()
        self.power, self.clk = [], []

    def run(self):
        cmd = ["amd-smi", "metric", "-g", str(self.gpu), "--power", "--clock", "--json"]
        while not self.halt.is_set():
            try:
                res = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
                data = json.loads(res.stdout)
                gd = data["gpu_data"][0] if isinstance(data, dict) else data[0]
                self.power.append(float(gd["power"]["socket_power"]["value"]))
                clks = [float(v["clk"]["value"]) for k, v in gd["clock"].items()
                        if k.startswith("gfx_") and isinstance(v, dict)
                        and isinstance(v.get("clk"), dict)]
                if clks:
                    self.clk.append(sum(clks) / len(clks))
            except Exception:
                return
            self.halt.wait(self.period)

    def summary(self):
        if not self.power:
            return None
        return {"source": "amd-smi metric during the timed steps", "samples": len(self.power),
                "socket_power_w_mean": round(sum(self.power) / len(self.power), 1),
                "gfx_clock_mhz_mean": round(sum(self.clk) / len(self.clk), 1) if self.clk
                else None}


def cpu_baseline(w, target_s: float = 15.0) -> dict:
    """The oracle's f-update on a sample of rows, scaled to iterations/s."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(0)
    g = np.zeros(w.m)
    k0 = min(w.n, 4 * oracle.num_threads())
    rows = rng.choice(w.n, size=k0, replace=False)
    t0 = time.perf_counter()
    oracle.f_update_rows(w.X, w.Y, w.b, g, w.eps, rows)
    t1 = time.perf_counter() - t0
    k = int(min(w.n, max(k0, round(k0 * target_s / max(t1, 1e-3)))))
    rows = rng.choice(w.n, size=k, replace=False)
    t0 = time.perf_counter()
    oracle.f_update_rows(w.X, w.Y, w.b, g, w.eps, rows)
    dt = time.perf_counter() - t0
    per_row = dt / k
    # one iteration = n row soft-mins (f-update) + m column soft-mins (g-update)
    iter_s = per_row * (w.n + w.m)
    return {"value": 1.0 / iter_s, "unit": "iters/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"float64 oracle f-update of {k} sampled rows of the {w.n} x {w.m}, "
                      f"d={w.d} workload ({dt:.1f} s); one iteration = {w.n + w.m} row "
                      f"soft-mins, so iters/s = 1 / ({w.n + w.m} x seconds per row)",
            "pair_evals_per_s": k * w.m / dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c3", choices=sorted(RECIPES))
    ap.add_argument("--prec", default=None,
                    choices=["auto", "fp32", "bf16", "fp16", "fp32-valu", "bf16-refine"],
                    help="override the recipe's score precision (the line then names it)")
    ap.add_argument("--iters", type=int, default=None, help="override iterations per stage")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hvp", action="store_true",
                    help="skip the Hessian-vector product measurement (d <= 64 recipes)")
    ap.add_argument("--pipeline-n", type=int, default=0,
                    help="fs2: also run the two-stage pipeline on two uniform clouds of this "
                         "many points at eps = n^(-2/3) (one dense iteration timed beside it)")
    ap.add_argument("--no-block-sparse", action="store_true",
                    help="skip the block-sparse measurement of the c5 line")
    ap.add_argument("--counters", action="store_true",
                    help="run the hardware-counter workload instead of the benchmark")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this solver has no multi-GPU path "
              "(its key ranges would shard across GPUs, but that is not built); "
              "run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from streaming_sinkhorn_solver_amd import binding, workloads

    binding.load()
    wl = args.workload
    prec, peak, unit, dtype, desc = RECIPES[wl]
    if args.prec and args.prec != prec:
        prec = args.prec
        dtype = {"bf16": "bf16", "fp16": "f16",
                 "bf16-refine": "bf16 (all but the last %d iteration(s)); f16 (those, "
                                "transport)" % max(REFINE_ITERS.get(wl, 0), 1)}.get(prec, "f32")
        desc += f" [score precision overridden: {prec}]"
    w = workloads.make(wl)
    if args.counters:
        counter_mode(w, prec)
        return
    if wl == "fs2":
        main_block_sparse(args, w, peak, unit, dtype, desc, binding, torch)
        return
    iters = args.iters or w.iters
    total_iters = iters * w.n_stages
    dev = torch.device("cuda:0")
    X = torch.from_numpy(w.X).to(dev)
    Y = torch.from_numpy(w.Y).to(dev)
    a = torch.from_numpy(w.a).to(dev)
    b = torch.from_numpy(w.b).to(dev)
    V = torch.from_numpy(w.V).to(dev) if w.V is not None else None
    dv = 0 if V is None else V.shape[1]
    f = torch.empty(w.n, device=dev)
    g = torch.empty(w.m, device=dev)
    U = torch.empty((w.n, dv), device=dev) if dv else None
    ws_bytes = binding.fs_workspace_bytes(w.n, w.m, w.d, dv, prec)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stats = {"lse_ms": 0.0, "lse_launches": 0, "init": 0.0, "solve": 0.0, "transport": 0.0}

    # the phase events of every step, created before the timed region
    ev_pool = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
               for _ in range(args.warmup + args.steps)]

    def step(timed: bool):
        ev = ev_pool.pop()
        ev[0].record()
        p = binding.fs_potentials_init(X, Y, a, b, dv_max=dv, prec=prec, f=f, g=g, workspace=ws)
        ev[1].record()
        # per-launch events from the library; a schedule that runs as one
        # launch is timed by the solve call's own events instead (the library's
        # timing waits for the launch, which would idle the device between steps)
        info = binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, eps_start=w.eps_start,
                                         n_stages=w.n_stages, iters_per_stage=iters,
                                         time_kernels=timed and not stats.get("single_launch"),
                                         refine_iters=REFINE_ITERS.get(wl, 0))
        ev[2].record()
        if dv:
            binding.fs_apply_transport(p, w.eps, f, g, V, U, divide_by_a=w.divide_by_a)
        ev[3].record()
        if timed:
            stats["lse_ms"] += info["lse_ms"]
            stats["lse_launches"] += info["lse_launches"]
            stats["events"].append(ev)
        stats["single_launch"] = info["single_launch"]
        return p

    stats["events"] = []

    for _ in range(args.warmup):
        p = step(False)
    torch.cuda.synchronize()
    sampler = PowerSampler()
    sampler.start()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        p = step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    sampler.halt.set()
    sampler.join(timeout=30)
    info = p.info

    for ev in stats["events"]:
        stats["init"] += ev[0].elapsed_time(ev[1])
        stats["solve"] += ev[1].elapsed_time(ev[2])
        stats["transport"] += ev[2].elapsed_time(ev[3])
    phases = {k: round(stats[k] / args.steps, 3) for k in ("init", "solve", "transport")}
    if stats.get("single_launch") and stats["lse_launches"] == 0:
        # one launch per solve: its half-steps are timed as the solve call
        # (the launch and one small fill kernel before it) over their number
        stats["lse_ms"] = stats["solve"]
        stats["lse_launches"] = 2 * total_iters * args.steps
    backward = None
    if dv >= w.d:
        # the backward pass of the end-to-end workload at the final
        # potentials: gradients with respect to both clouds (outside the
        # timed steps; one untimed call first)
        gX = torch.empty((w.n, w.d), device=dev)
        gY = torch.empty((w.m, w.d), device=dev)
        binding.fs_gradient(p, w.eps, f, g, X, Y, gX, gY)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        binding.fs_gradient(p, w.eps, f, g, X, Y, gX, gY)
        e1.record()
        torch.cuda.synchronize()
        backward = {"gradient_ms": round(e0.elapsed_time(e1), 3),
                    "what": "fs_gradient for both clouds at the final potentials (two transport "
                            "applications of width d, each also leaving its rows' LSE2 for "
                            "the finishing pass)"}
        del gX, gY

    hvp = None
    fused_moment = prec in ("bf16", "fp16") and 64 <= w.d <= 512
    if (w.d <= 64 or fused_moment) and not args.no_hvp:
        # the streaming Hessian-vector product at the final potentials (its
        # own problem handle: it needs dv_max >= d + 2; without the one-pass
        # second-moment kernel it runs the d*d moment columns in passes of
        # dv_max, one pass when dv_max >= d*d); outside the timed steps, one
        # untimed call first
        hdv = w.d + 2 if fused_moment else max(w.d + 2, min(w.d * w.d, 4096))
        hws = torch.empty(binding.fs_workspace_bytes(w.n, w.m, w.d, hdv, prec) + 256,
                          dtype=torch.uint8, device=dev)
        fh, gh = torch.empty_like(f), torch.empty_like(g)
        ph = binding.fs_potentials_init(X, Y, a, b, dv_max=hdv, prec=prec, f=fh, g=gh,
                                        workspace=hws)
        fh.copy_(f)
        gh.copy_(g)
        Vd = torch.from_numpy(np.random.default_rng(7).standard_normal((w.n, w.d))
                              .astype(np.float32)).to(dev)
        HV = torch.empty_like(Vd)
        scratch = torch.empty(binding.fs_hvp_workspace_bytes(ph), dtype=torch.uint8, device=dev)
        binding.fs_hvp(ph, w.eps, fh, gh, X, Y, Vd, HV, workspace=scratch)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        hinfo = binding.fs_hvp(ph, w.eps, fh, gh, X, Y, Vd, HV, workspace=scratch)
        torch.cuda.synchronize()
        hvp = {"hvp_ms": round((time.perf_counter() - t1) * 1e3, 3), **hinfo,
               "what": "fs_hvp at the final potentials, random direction, CG to 1e-4 "
                       "(two LSE passes; transports of widths d, d+2, d+1, two of width 1 "
                       "per CG step, and the second moment: one pass with the direction "
                       "rows as a second resident block"
                       + (")" if fused_moment else " replaced by d*d columns in passes)")}
        del hws, scratch, HV, Vd, ph

    ms_per_step = dt / args.steps * 1e3
    it_s = total_iters * args.steps / dt
    pair_evals = 2.0 * w.n * w.m * total_iters * args.steps
    lse_mean_ms = stats["lse_ms"] / max(stats["lse_launches"], 1)
    # the LSE launches alternate f (n rows) and g (m rows); per launch the
    # same n*m pairs
    if unit == "TFLOP/s":
        work = 2.0 * w.n * w.m * w.d  # score contraction flops of one half-step
    else:
        work = float(w.n) * w.m  # exponentials of one half-step
    achieved = work / (lse_mean_ms * 1e-3) / 1e12
    kernel = {"c1": "lse_small_kernel<2> (fp16 split scores)",
              "c5": "lse_small_kernel<2> (fp16 split scores)",
              "c2": "lse_mfma_kernel<fp32, d_pad 64>",
              "c3": "lse_mfma_kernel<%s, d_pad 512>" % ("bf16" if prec == "bf16-refine"
                                                         else prec),
              "c4": "lse_wide_kernel<%s> (1024-wide rows, contraction split over wave pairs)"
                    % ("bf16 in stages 1-9, fp16 in stage 10" if prec == "bf16-refine"
                       else prec)}[wl]
    kernel += " (one half-step)"
    if stats.get("single_launch"):
        # one launch runs the whole schedule; its half-steps are reported as
        # the launch's duration over their number
        kernel = ("solve_persistent_kernel<%d> (one launch runs all %d half-steps, fp32 "
                  "scores; per half-step: the event-timed solve call, i.e. the launch and "
                  "one small fill kernel, / %d)" % (w.d, 2 * total_iters, 2 * total_iters))
    sink = torch.zeros(1, device=dev)
    probe = {"bf16": "mfma-bf16", "bf16-refine": "mfma-bf16",
             "fp16": "mfma-fp16"}.get(prec, PROBES[wl]) \
        if unit == "TFLOP/s" and prec != "fp32" else PROBES[wl]
    peak_measured = binding.fs_probe_peak(probe, sink) / 1e12
    roofline = {"bound": "mfma" if unit == "TFLOP/s" else "alu",
                "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic_per_launch(wl),
                "peak_measured": round(peak_measured, 2),
                "frac_measured": round(achieved / peak_measured, 4),
                "peak_probe": probe,
                "kernel": kernel,
                "mean_launch_ms": round(lse_mean_ms, 4), "launches": stats["lse_launches"]}
    clocks = sampler.summary()
    if stats.get("single_launch"):
        dtype = "f32"
    elif info["path"] == "fp32-small-mfma":
        dtype = small_path_dtype(w.X, w.Y, w.a, w.b, f.cpu().numpy(), g.cpu().numpy(), w.eps)
    out = {
        "metric": METRIC, "value": round(it_s, 3), "unit": "iters/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": desc, "recipe": wl, "n": w.n, "m": w.m, "d": w.d,
                   "eps": w.eps, "eps_start": w.eps_start, "n_stages": w.n_stages,
                   "iters_per_stage": iters, "transport_width": dv,
                   "score_path": info["path"], "f_splits": info["f_splits"],
                   "g_splits": info["g_splits"]},
        "pair_evals_per_s": pair_evals / dt,
        "phases_ms": phases,
        "clocks": clocks,
        "roofline": roofline,
    }
    if dv and unit == "TFLOP/s" and phases["transport"] > 0:
        # the transport phase (every launch of one application) against the
        # matrix peak: 2 n m (d + dv) algorithmic flops
        t_flops = 2.0 * w.n * w.m * (w.d + dv)
        t_ach = t_flops / (phases["transport"] * 1e-3) / 1e12
        out["transport_roofline"] = {
            "bound": "mfma", "flops": t_flops, "achieved": round(t_ach, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(t_ach / peak, 4),
            "what": "phases_ms.transport (all launches of one application, event-timed) "
                    "against 2 n m (d + dv) flops"}
    if backward:
        out["backward"] = backward
    if hvp:
        out["hvp"] = hvp
    if wl == "c5" and not args.no_block_sparse:
        out["block_sparse"] = block_sparse_run(w, w.eps, 3, 1, dev, binding, torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


def fs2_pipeline(w, dev, binding, torch, cell=8, tol=1e-2, max_iters=3000, dense_full=True,
                 coarse_delta=0.0):
    """The whole two-stage solve on the workload (outside the timed steps):
    Morton order, the coarse stage (centroids of `cell` points, a dense solve
    on them annealed 0.1 -> eps, lift, sampled check on 1024 rows and columns,
    at most 2 rounds), then block-sparse iterations at eps from the lift until
    the L1 marginal residual of the retained blocks' plan is at most `tol`
    (checked every 10 iterations).  coarse_delta > 0 runs the coarse solve in
    block-sparse form.  Beside it the dense path from the same lift: to the
    same target (dense_full), else one timed dense iteration."""
    import numpy as np

    X = torch.from_numpy(w.X).to(dev)
    Y = torch.from_numpy(w.Y).to(dev)
    a = torch.from_numpy(w.a).to(dev)
    b = torch.from_numpy(w.b).to(dev)
    rng = np.random.default_rng(11)
    rows = torch.from_numpy(rng.choice(w.n, 1024, replace=False).astype(np.int32)).to(dev)
    cols = torch.from_numpy(rng.choice(w.m, 1024, replace=False).astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Xs, a_s, _ = binding.fs_morton_sort(X, a)
    Ys, b_s, _ = binding.fs_morton_sort(Y, b)
    CX, WX = binding.fs_centroids(Xs, a_s, cell)
    CY, WY = binding.fs_centroids(Ys, b_s, cell)
    F = torch.empty(CX.shape[0], device=dev)
    G = torch.empty(CY.shape[0], device=dev)
    pc = binding.fs_potentials_init(CX, CY, WX, WY, f=F, g=G)
    if coarse_delta > 0:
        binding.fs_bs_attach(pc)
    f = torch.empty(w.n, device=dev)
    g = torch.empty(w.m, device=dev)
    cinfo = binding.fs_bs_coarse_start(pc, Xs, Ys, a_s, b_s, cell, f, g, F, G, rows, cols,
                                       eps_end=w.eps, eps_start=0.1, n_stages=12,
                                       iters_per_stage=10, more_iters=20, check_tol=0.5,
                                       max_rounds=2, coarse_delta=coarse_delta)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    f_lift, g_lift = f.clone(), g.clone()
    p = binding.fs_potentials_init(Xs, Ys, a_s, b_s)
    binding.fs_bs_attach(p)
    info = binding.fs_bs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=max_iters,
                                        delta=BS_DELTA, tol=tol, check_every=10, warm_start=True,
                                        raise_not_converged=False)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    res = torch.zeros(2, device=dev)
    binding.fs_marginal_residual(p, w.eps, f, g, res)
    r = res.cpu().numpy()
    # the dense path from the same lift to the same target
    t3 = time.perf_counter()
    dinfo = binding.fs_sinkhorn_solve(p, f_lift, g_lift, eps_end=w.eps,
                                      iters_per_stage=max_iters if dense_full else 1,
                                      tol=tol if dense_full else 0.0, check_every=10,
                                      warm_start=True, raise_not_converged=False)
    torch.cuda.synchronize()
    t4 = time.perf_counter()
    dense = ({"dense_fine_iters": dinfo["iters_done"], "dense_fine_ms": round((t4 - t3) * 1e3, 3)}
             if dense_full else {"dense_ms_per_iter": round((t4 - t3) * 1e3, 3)})
    return {"n": w.n, "m": w.m, "eps": w.eps, "cell": cell, "coarse_delta": coarse_delta,
            "coarse_points": [int(CX.shape[0]), int(CY.shape[0])], **dense,
            "coarse_ms": round((t1 - t0) * 1e3, 3), "coarse": cinfo,
            "fine_iters": info["iters_done"], "fine_ms": round((t2 - t1) * 1e3, 3),
            "fine_residual_retained": info["residual"],
            "dense_residual_after": [float(r[0]), float(r[1])],
            "total_ms": round((t2 - t0) * 1e3, 3), "target_residual": tol,
            "what": "Morton order + coarse stage (solve on centroids, block-sparse when "
                    "coarse_delta > 0, lift, sampled check) + block-sparse iterations from "
                    "the lift to an L1 marginal "
                    "residual <= target (wall clock, including the set-up)"}


def main_block_sparse(args, w, peak, unit, dtype, desc, binding, torch):
    from streaming_sinkhorn_solver_amd import workloads

    dev = torch.device("cuda:0")
    sampler = PowerSampler()
    sampler.start()
    bs = block_sparse_run(w, w.eps, args.steps, args.warmup, dev, binding, torch)
    sampler.halt.set()
    sampler.join(timeout=30)
    sink = torch.zeros(1, device=dev)
    peak_measured = binding.fs_probe_peak("exp", sink) / 1e12
    # one exponential per kept pair; launches alternate the two sides
    achieved = bs["kept_pairs_per_iter"] / 2 / (bs["lse_mean_launch_ms"] * 1e-3) / 1e12
    roofline = {"bound": "alu", "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic_per_launch("fs2"),
                "peak_measured": round(peak_measured, 2),
                "frac_measured": round(achieved / peak_measured, 4), "peak_probe": "exp",
                "kernel": "lse_small_kernel<2, sparse> (one half-step; work = exponentials of "
                          "the kept 32 x 256 block pairs)",
                "mean_launch_ms": bs["lse_mean_launch_ms"], "launches": bs["lse_launches"]}
    it_s = bs["iters_per_s"]
    out = {
        "metric": METRIC, "value": it_s, "unit": "iters/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(10e3 / it_s, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16x3-split/f32-acc (f16x3-split/f32-acc in a pass or row block whose "
                 "fp16 guard holds)",
        "data": "synthetic",
        "config": {"workload": desc, "recipe": "fs2", "n": w.n, "m": w.m, "d": w.d,
                   "eps": w.eps, "delta": BS_DELTA, "iters_per_step": 10,
                   "score_path": "small-mfma (block-sparse)"},
        "pair_evals_per_s": bs["kept_pairs_per_iter"] * it_s,
        "dense_equivalent_pair_evals_per_s": 2.0 * w.n * w.m * it_s,
        "clocks": sampler.summary(),
        "roofline": roofline,
        "block_sparse": bs,
        "pipeline": fs2_pipeline(w, dev, binding, torch, coarse_delta=BS_DELTA),
        # cells of 16 points: the fastest of 4, 8, 16 and 32 on two 2M-point clouds
        **({"pipeline_large": fs2_pipeline(
            workloads.make("fs2", n=args.pipeline_n, m=args.pipeline_n), dev, binding, torch,
            cell=16, dense_full=False, coarse_delta=BS_DELTA)} if args.pipeline_n else {}),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block_sparse(w, bs)
    print(json.dumps(out), flush=True)


def cpu_baseline_block_sparse(w, bs, row_blocks=(0, 1)) -> dict:
    """The block-sparse oracle (oracle/blocksparse.py, numpy) on two row
    blocks of the f-update at the warm start's final eps, from zero
    potentials (its screening of those blocks plus their retained-block
    LSE), scaled to iterations per second of the whole problem."""
    import numpy as np

    from oracle import blocksparse as obs

    X = w.X[obs.morton_order(w.X)]
    Y = w.Y[obs.morton_order(w.Y)]
    t = time.perf_counter()
    obs.update_sparse(X, Y, w.b, np.zeros(w.m), np.zeros(w.n), w.eps, BS_DELTA,
                      row_blocks=list(row_blocks))
    dt = time.perf_counter() - t
    rows = 256 * len(row_blocks)
    per_half = dt * w.n / rows
    return {"value": round(1.0 / (2 * per_half), 6), "unit": "iters/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle/blocksparse.py update_sparse on {len(row_blocks)} row blocks "
                      f"({rows} rows; screening against all key blocks, then the retained "
                      f"blocks' LSE) of the f-update from zero potentials at eps={w.eps:.3g}, "
                      f"{dt:.1f} s, scaled to both half-steps of all rows"}


if __name__ == "__main__":
    main()
