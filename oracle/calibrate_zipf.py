"""Calibrate the Zipf logit-offset scale of the skewed workload with the oracle's router.

TEST INFRASTRUCTURE.  The skewed workload adds o_e = -s * a * ln(rank_e) to the routed
experts' logits.  This script finds ``a`` by bisection, on the workload's own seeded
inputs, so that the 8 hottest experts (ranks 1..8) receive the target share of all
routed assignments (0.30 +- 0.005), and writes it to moe_inputs/zipf_calibration.json.
The routing is the oracle's; nothing here touches the GPU library.

Run:  python -m oracle.calibrate_zipf
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from moe_inputs import CONFIGS  # noqa: E402
from moe_inputs.generate import (  # noqa: E402
    _CALIB_FILE, make_sel_bias, make_w_router, make_x, zipf_ranks)
from oracle.moe_oracle import promote, route_sigmoid_shared, router_logits  # noqa: E402


def hot_share(cfg, logits0, bias, ranks, a):
    off = -cfg.zipf_s * a * np.log(ranks.astype(np.float64))
    off = off.astype(np.float32).astype(np.float64)     # the generator stores float32
    l = logits0.copy()
    l[:, :cfg.E] += off
    r = route_sigmoid_shared(l, cfg.E, cfg.S, cfg.k, cfg.route_scale, bias,
                             cfg.bias_on_logits)
    hot = np.nonzero(ranks <= 8)[0]
    return r.counts[hot].sum() / (cfg.T * cfg.k)


def calibrate(name: str, tol: float = 0.005):
    cfg = CONFIGS[name]
    logits0 = router_logits(promote(make_x(cfg), cfg.dtype),
                            promote(make_w_router(cfg), cfg.dtype), cfg.E)
    bias = make_sel_bias(cfg)
    ranks = zipf_ranks(cfg)
    lo, hi = 0.0, 4.0
    target = cfg.zipf_hot_share
    a = share = None
    for _ in range(60):
        a = 0.5 * (lo + hi)
        share = hot_share(cfg, logits0, bias, ranks, a)
        print(f"  a={a:.6f} hot-8 share={share:.5f}", flush=True)
        if abs(share - target) <= tol / 4:
            break
        if share < target:
            lo = a
        else:
            hi = a
    assert abs(share - target) <= tol, (a, share)
    return {"a": a, "hot8_share": share, "target": target, "tolerance": tol,
            "seed": cfg.seed, "T": cfg.T}


def main():
    table = {}
    if os.path.exists(_CALIB_FILE):
        with open(_CALIB_FILE) as f:
            table = json.load(f)
    for name, cfg in CONFIGS.items():
        if cfg.zipf_s:
            print(f"calibrating {name}", flush=True)
            table[name] = calibrate(name)
    with open(_CALIB_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(table, indent=1))


if __name__ == "__main__":
    main()
