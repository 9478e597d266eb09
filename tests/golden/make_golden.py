"""Write the stored oracle outputs under tests/golden/.

Calls only ``oracle/`` (and the shared seeded input generator).  The pages
(FlashSinkhorn explainer) print no potential, plan or worked example, so no
fixture here comes from the pages; these files are snapshots of the float64
oracle on the 512 x 512, 3-D recipe (eps 0.1, uniform weights), used as the
expected values of the GPU parity test for that recipe and as a regression
check of the oracle itself.  Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from streaming_sinkhorn_solver_amd import workloads  # noqa: E402


def main():
    w = workloads.make("c1")
    for iters in (1, 100):
        res = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=iters)
        for key in ("f", "g"):
            path = os.path.join(HERE, f"c1_oracle_{key}_iter{iters}.txt")
            np.savetxt(path, res[key], fmt="%.17e",
                       header=f"oracle v{oracle.version()} c1 seed 1 eps {w.eps} "
                              f"iterations {iters} potential {key}")
    res = oracle.sinkhorn(w.X, w.Y, w.a, w.b, eps=w.eps, iters=100)
    tot, rt, ct = oracle.marginal_residual(w.X, w.Y, w.a, w.b, res["f"], res["g"], w.eps)
    np.savetxt(os.path.join(HERE, "c1_oracle_residual_iter100.txt"), [tot, rt, ct],
               fmt="%.17e", header="total, row term, column term of the L1 marginal residual")


if __name__ == "__main__":
    main()
