"""Write the full-size, full-schedule oracle outputs of the five recipes.

Calls only ``oracle/`` and the shared seeded input generator (never the HIP
path).  The pages (FlashSinkhorn explainer, "Method" and "Experimental
results") print no potential or plan, so these files are snapshots of the
float64 oracle, used as the expected values of the full-size GPU parity
tests (``tests/test_fullsize_schedule_gpu.py``).

Per recipe, at its real shape and over its whole schedule from g = 0:

  c2  10k x 10k x 64, eps 0.05, 200 iterations: f, g and the L1 marginal
      residual (direct-difference oracle, ``oracle.c``);
  c3  50k x 50k x 512, eps 0.1, 100 iterations: f, g, and the barycentric
      projection T = P.Y / a of 512 seeded rows;
  c4  50k x 30k x 1024, eps 1 -> 0.01 over 10 stages x 20 iterations: f, g,
      and U = P.V of 512 seeded rows;
  c5  250k x 250k x 3, eps 0.01, 10 iterations: f, g (``oracle.c``).

c3 and c4 iterate with ``oracle/expanded.py`` (the same update with the dot
products from a float64 matrix product: the direct-difference oracle needs
about 200 s per c3 half-step on 8 cores).  Each of their files records the
largest difference, on 256 seeded rows and columns, between that iteration
and the direct-difference oracle's update from the same potentials, at the
first and at the last iteration; the script refuses to write a file where it
exceeds 1e-9 eps.  Their transports are evaluated by the direct-difference
oracle at the final potentials.

Run (hours of CPU for c3 and c4):  python tests/golden/make_golden_full.py c2 c3 c4 c5
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from oracle import expanded  # noqa: E402
from streaming_sinkhorn_solver_amd import workloads  # noqa: E402

N_SAMPLE_OUT = 512  # rows of the stored transport
N_SAMPLE_PIN = 256  # rows / columns of the direct-difference cross-check
PIN_BAR = 1e-9  # largest allowed |expanded - direct| / eps


def sample_rows(seed: int, count: int, k: int) -> np.ndarray:
    """Seeded sorted sample of k distinct indices in [0, count)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(count, size=min(k, count), replace=False)).astype(np.int64)


def out_path(name: str) -> str:
    return os.path.join(HERE, f"{name}_oracle_full.npz")


def write(name: str, arrays: dict, meta: dict) -> None:
    np.savez_compressed(out_path(name), **arrays)
    with open(os.path.join(HERE, f"{name}_oracle_full.json"), "w") as fh:
        json.dump(meta, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(f"[golden] wrote {name}: {json.dumps(meta)}", flush=True)


def direct(name: str) -> None:
    """c2, c5: the direct-difference oracle over the whole schedule."""
    w = workloads.make(name)
    t0 = time.time()
    res = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=w.iters,
                          n_stages=w.n_stages, eps_start=w.eps_start)
    meta = {"recipe": name, "seed": w.seed, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps,
            "iterations": res["iters"], "oracle": f"oracle.c v{oracle.version()}",
            "threads": oracle.num_threads(), "seconds": round(time.time() - t0, 1)}
    arrays = {"f": res["f"], "g": res["g"]}
    if name == "c2":
        tot, rt, ct = oracle.marginal_residual(w.X, w.Y, w.a, w.b, res["f"], res["g"], w.eps)
        arrays["residual"] = np.array([tot, rt, ct])
    write(name, arrays, meta)


def gemm(name: str) -> None:
    """c3, c4: the matrix-product form, cross-checked against oracle.c."""
    w = workloads.make(name)
    total = w.iters * w.n_stages
    pin_rows = sample_rows(2000 + w.seed, w.n, N_SAMPLE_PIN)
    pin_cols = sample_rows(3000 + w.seed, w.m, N_SAMPLE_PIN)
    state = {"g_prev": np.zeros(w.m), "pins": [], "t0": time.time()}

    def on_iteration(k, e, f, g):
        if k in (1, total):
            fr = oracle.f_update_rows(w.X, w.Y, w.b, state["g_prev"], e, pin_rows)
            gc = oracle.g_update_cols(w.X, w.Y, w.a, f, e, pin_cols)
            df = float(np.abs(fr - f[pin_rows]).max() / e)
            dg = float(np.abs(gc - g[pin_cols]).max() / e)
            state["pins"].append({"iteration": k, "eps": e, "max_df_over_eps": df,
                                  "max_dg_over_eps": dg})
            if max(df, dg) > PIN_BAR:
                raise SystemExit(f"{name}: expanded form differs from oracle.c by "
                                 f"{max(df, dg):.3e} eps at iteration {k}")
        state["g_prev"] = g.copy()
        if k % 10 == 0 or k == 1:
            print(f"[golden] {name} iteration {k}/{total} eps {e:.4g} "
                  f"({time.time() - state['t0']:.0f} s)", flush=True)

    res = expanded.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=w.iters,
                            n_stages=w.n_stages, eps_start=w.eps_start,
                            on_iteration=on_iteration)
    seconds = time.time() - state["t0"]
    rows = sample_rows(1000 + w.seed, w.n, N_SAMPLE_OUT)
    U = oracle.transport(w.X, w.Y, w.a, w.b, res["f"], res["g"], w.V, w.eps,
                         divide_by_a=w.divide_by_a, rows=rows)
    meta = {"recipe": name, "seed": w.seed, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps,
            "eps_start": w.eps_start, "n_stages": w.n_stages, "iters_per_stage": w.iters,
            "iterations": res["iters"], "oracle": "oracle/expanded.py (float64 matmul form)",
            "transport": f"oracle.c v{oracle.version()} transport of {len(rows)} rows, "
                         f"divide_by_a={bool(w.divide_by_a)}",
            "pins_vs_direct_difference": state["pins"], "seconds": round(seconds, 1)}
    write(name, {"f": res["f"], "g": res["g"], "rows": rows, "U_rows": U}, meta)


def main(names):
    for name in names:
        if name in ("c2", "c5"):
            direct(name)
        elif name in ("c3", "c4"):
            gemm(name)
        else:
            raise SystemExit(f"unknown recipe {name}")


if __name__ == "__main__":
    main(sys.argv[1:] or ["c2", "c3", "c4", "c5"])
