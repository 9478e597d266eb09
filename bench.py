#!/usr/bin/env python3
"""Benchmark of the streaming log-domain Sinkhorn solver on one MI355X.

Workload (the recipe the headline metric is quoted on): n = m = 50,000
points in 512-D, two 10-component Gaussian mixtures, Dirichlet(1) weights,
eps = 0.1, bf16 matrix-core scores with fp32 accumulation.  One step is the
whole hot path on resident inputs: problem preparation (shift, bf16
conversion, norms, log-weights), 100 alternating f/g iterations and the
barycentric projection P.Y / a.

Prints one JSON line with
  value      Sinkhorn iterations per second over whole steps
  roofline   the streaming LSE kernel: algorithmic flops per launch
             (2 n m d) over its mean launch duration, timed with HIP events
             on the launch stream inside the timed region, against the
             MI355X dense bf16 peak; `traffic` is the per-launch HBM bytes
             from the committed rocprofv3 counter summary when it was taken
             on the current kernel source, else null
  cpu_baseline  the float64 oracle's f-update timed on this host's cores
             on a bounded sample of rows of the same workload, scaled to
             iterations per second
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "Sinkhorn iters/sec and pair-evals/sec at n=m=50k, d=512; % of roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
TRAFFIC_FILE = os.path.join(HERE, "profiles", "lse_bf16_c3_traffic.json")
KERNEL_SOURCE = os.path.join(HERE, "streaming_sinkhorn_solver_amd", "csrc", "fs_lse.hip")


def kernel_source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def counter_mode(w, half_steps: int = 6) -> None:
    """Workload for hardware-counter runs: a 1 GiB elementwise read+write of
    known size (the counters' calibration), then problem preparation and
    `half_steps` alternating LSE passes of the benchmark workload."""
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
    p = binding.fs_potentials_init(X, Y, a, b, prec="bf16", f=f, g=g)
    for k in range(half_steps):
        if k % 2 == 0:
            binding.fs_lse_update_f(p, w.eps, g, f)
        else:
            binding.fs_lse_update_g(p, w.eps, f, g)
    torch.cuda.synchronize()
    print(json.dumps({"counter_mode": "done", "half_steps": half_steps,
                      "copy_bytes": float(1 << 30)}), flush=True)


def traffic_per_launch():
    """Calibrated HBM bytes per LSE launch from the committed counter summary,
    or None if it is missing or was taken on another kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, target_s: float = 15.0) -> dict:
    """The oracle's f-update on a sample of rows, scaled to iterations/s."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(0)
    g = np.zeros(w.m)
    k0 = 4 * oracle.num_threads()
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
    ap.add_argument("--iters", type=int, default=None, help="override iterations per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="run the hardware-counter workload instead of the benchmark")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this solver has no multi-GPU path "
              "(the sharding design is described in DESIGN.md); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from streaming_sinkhorn_solver_amd import binding, workloads

    binding.load()
    w = workloads.make("c3")
    if args.counters:
        counter_mode(w)
        return
    iters = args.iters or w.iters
    dev = torch.device("cuda:0")
    X = torch.from_numpy(w.X).to(dev)
    Y = torch.from_numpy(w.Y).to(dev)
    a = torch.from_numpy(w.a).to(dev)
    b = torch.from_numpy(w.b).to(dev)
    V = Y  # barycentric projection of the target cloud
    f = torch.empty(w.n, device=dev)
    g = torch.empty(w.m, device=dev)
    T = torch.empty((w.n, w.d), device=dev)
    ws_bytes = binding.fs_workspace_bytes(w.n, w.m, w.d, w.d, "bf16")
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stats = {"lse_ms": 0.0, "lse_launches": 0}

    def step(timed: bool):
        p = binding.fs_potentials_init(X, Y, a, b, dv_max=w.d, prec="bf16", f=f, g=g,
                                       workspace=ws)
        info = binding.fs_sinkhorn_solve(p, f, g, eps_end=w.eps, iters_per_stage=iters,
                                         time_kernels=timed)
        binding.fs_apply_transport(p, w.eps, f, g, V, T, divide_by_a=True)
        if timed:
            stats["lse_ms"] += info["lse_ms"]
            stats["lse_launches"] += info["lse_launches"]
        return p

    for _ in range(args.warmup):
        p = step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        p = step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    info = p.info

    total_iters = iters * args.steps
    ms_per_step = dt / args.steps * 1e3
    it_s = total_iters / dt
    pair_evals = 2.0 * w.n * w.m * total_iters
    flops_per_launch = 2.0 * w.n * w.m * w.d  # score contraction of one half-step
    lse_mean_ms = stats["lse_ms"] / max(stats["lse_launches"], 1)
    achieved = flops_per_launch / (lse_mean_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_per_launch(),
                "kernel": "lse_mfma_kernel<bf16, d_pad 512> (one half-step)",
                "mean_launch_ms": round(lse_mean_ms, 4), "launches": stats["lse_launches"]}
    out = {
        "metric": METRIC, "value": round(it_s, 3), "unit": "iters/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "n=m=50000, d=512, two 10-component Gaussian mixtures, "
                               "Dirichlet(1) weights, eps=0.1, 100 alternating iterations + "
                               "barycentric projection P.Y/a (seed 3)",
                   "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "iters_per_step": iters,
                   "score_path": info["path"], "f_splits": info["f_splits"],
                   "g_splits": info["g_splits"]},
        "pair_evals_per_s": pair_evals / dt,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
