"""Write skewed_router_bias.json: the fp32 router bias that gives the skewed workload its expert loads.

The skewed workload (T=65536, d_model=2048, 8 experts, no load-balancing loss) asks for expert loads of
60/10/10/5/5/5/3/2 %. The router's fp32 logits are shifted by a per-expert bias b, calibrated on the
workload's own seeded X and W_router with the CPU oracle's router only:
    b <- b + eta * log(target / observed),  eta = 0.4
(at most 200 rounds, stop once every load is within 0.25 points of its target). The damping eta is about
the Gumbel scale that the maximum of 8 Gaussian logits of std ~0.9 behaves like; eta = 1 oscillates.
Run from the repository root:  python tests/golden/make_skewed_router_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.WORKLOADS["skewed"]
    inp = workloads.make_inputs(w, router_bias=np.zeros(w.E, np.float32), which={"X", "W_router"})
    target = np.array(w.skew, np.float64)
    orc = oracle.default()
    b = np.zeros(w.E, np.float32)
    for it in range(200):
        ids = orc.route(inp["X"], inp["W_router"], b)["ids"][:, 0]
        frac = np.bincount(ids, minlength=w.E) / w.T
        print(f"round {it}: loads % = {np.round(100 * frac, 3).tolist()}", flush=True)
        if np.max(np.abs(frac - target)) <= 0.0025:
            break
        b = (b.astype(np.float64) + 0.4 * np.log(target / np.maximum(frac, 1.0 / w.T))).astype(np.float32)
    else:
        raise SystemExit("calibration did not converge")
    counts = np.bincount(ids, minlength=w.E)
    rec = dict(workload=w.name, seed=w.seed, T=w.T, d_model=w.d_model, E=w.E,
               target_loads=list(w.skew), bias=[float(v) for v in b], counts=counts.tolist(),
               note="written by make_skewed_router_bias.py with the CPU oracle's router; an input, not an expected value")
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "skewed_router_bias.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
