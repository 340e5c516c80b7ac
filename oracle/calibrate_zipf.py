"""Calibrate the Zipf logit-offset scale alpha of the skewed-capacity workload.

Test infrastructure: it runs the CPU oracle's router on the seed-0 inputs and bisects alpha so that
the hottest expert's load max_e n_e is about 8x the mean load k T / E, then writes
``workloads/zipf_alpha.json``. The stored alpha is an input-generation constant; no expected value
of any test is derived from it.

    python oracle/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workloads  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

TARGET = 8.0


def hot_ratio(cfg, x64, alpha):
    W_r = O._f64(workloads.make_router(cfg, alpha))
    r = O.route(x64, W_r, cfg.k)
    n = O.expert_loads(r["topk_idx"], cfg.E)
    return n.max() / (cfg.k * cfg.T / cfg.E), n


def main():
    cfg = workloads.CONFIGS["skewed_capacity"]
    x64 = O._f64(workloads.make_x(cfg))
    lo, hi = 0.0, 4.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        ratio, _ = hot_ratio(cfg, x64, mid)
        if ratio < TARGET:
            lo = mid
        else:
            hi = mid
        print(f"alpha={mid:.6f} hottest/mean={ratio:.3f}", flush=True)
        if abs(ratio - TARGET) < 0.05:
            break
    alpha = round(mid, 6)
    ratio, n = hot_ratio(cfg, x64, alpha)
    path = os.path.join(os.path.dirname(workloads.__file__), "zipf_alpha.json")
    table = {}
    if os.path.exists(path):
        with open(path) as fh:
            table = json.load(fh)
    table[f"{cfg.name}:s={cfg.zipf_s}"] = {
        "alpha": alpha, "seed": cfg.seed, "hottest_over_mean": float(ratio),
        "max_load": int(n.max()), "min_load": int(n.min()),
        "written_by": "oracle/calibrate_zipf.py"}
    with open(path, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    print(json.dumps(table, indent=1))


if __name__ == "__main__":
    main()
