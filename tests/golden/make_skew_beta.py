"""Writes skew_beta.json: the hot-centroid alignment strength beta of the
skewed-load workload (T=16384, d_model=7168, E_r=256, K=8, 4-component token
mixture, 8 hot experts), chosen by bisection so that the hot experts take
50% +- 1% of the T*K assignments at step 0 under the oracle's routing with
b = 0.  Calls only the input generators and the oracle:

    python tests/golden/make_skew_beta.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402
from synthetic import CONFIGS, host_array, make_tokens  # noqa: E402
from synthetic.gen import make_centroids  # noqa: E402


def hot_share(cfg, h, beta):
    e = host_array(make_centroids(cfg, beta=beta))
    r = O.route(h, e, np.zeros(cfg.E_r, np.float32), cfg.K, cfg.score)
    return r["loads"][:cfg.hot_experts].sum() / (cfg.T * cfg.K), r


def main():
    cfg = CONFIGS["dsv3_skewed"]
    h = host_array(make_tokens(cfg, step=0))
    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        share, _ = hot_share(cfg, h, mid)
        print(f"beta={mid:.6f} hot share={share:.4f}", flush=True)
        if abs(share - 0.5) <= 0.002:
            break
        if share < 0.5:
            lo = mid
        else:
            hi = mid
    share, r = hot_share(cfg, h, mid)
    c = r["loads"]
    out = dict(
        source="Bisection on the oracle's step-0 routing of the skewed workload (b = 0); "
               "target: hot experts take 50% of the T*K assignments.",
        beta=round(mid, 6), hot_share=float(share), max_load=int(c.max()), min_load=int(c.min()),
        max_vio=float(O.max_vio(c, cfg.T, cfg.K)))
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_beta.json"), "w") as f:
        json.dump(out, f, indent=2)
    print(out)


if __name__ == "__main__":
    main()
