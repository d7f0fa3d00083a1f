"""Write tests/golden/c2_rho.json: the row correlation of the 8-row similar-rows workload.

Rows are x = sqrt(rho) z0 + sqrt(1-rho) z_row.  rho is found by bisection so
that the oracle's routing of the 8 rows (each redrawn until its top-k is well
posed, as the tests draw them) repeats an expert in 30 % of the 80 picks:
repeat fraction = 1 - distinct / (R K).  Calls only the oracle.

    python tests/golden/make_c2_rho.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from cases import gapped_rows  # noqa: E402
from decode_moe_layer_amd import synth  # noqa: E402

TARGET = 0.30


def repeat_fraction(cfg, rw, rho):
    x, r, attempts = gapped_rows(cfg, rw, rho=rho)
    _, ky = oracle.router_keys(x, r, rw, cfg)
    picks = np.concatenate([oracle.topk(ky[i], cfg.topk) for i in range(cfg.rows)])
    return 1.0 - len(set(picks.tolist())) / picks.size, attempts


def main():
    cfg = synth.CONFIGS["c2"]
    rw = synth.make_router_weights(cfg)
    lo, hi = 0.0, 1.0
    best = None
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        f, att = repeat_fraction(cfg, rw, mid)
        if best is None or abs(f - TARGET) < abs(best[1] - TARGET):
            best = (mid, f, att)
        if abs(f - TARGET) <= 0.0125:
            break
        if f < TARGET:
            lo = mid
        else:
            hi = mid
    rho, f, att = best
    out = {"rho": round(rho, 6), "repeat_fraction": f, "attempts": att, "target": TARGET,
           "note": "written by tests/golden/make_c2_rho.py from the oracle's routing"}
    with open(os.path.join(HERE, "c2_rho.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(out)


if __name__ == "__main__":
    main()
