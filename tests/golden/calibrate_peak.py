"""Choose the planted-peak strength of the synthetic workloads.

The SpeCache summary (§2, "attention sparsity" with Figure 2 left) reports that
0.5% of the keys carry about 90% of a query's attention.  The synthetic caches
plant ceil(0.005 N) keys per slice along a unit direction u and add peak * u to
the queries of that KV head; this script finds, by bisection, the `peak` for
which the speculative row's float64 attention over the 16-bit cache puts 90%
of its mass on the planted keys (mean over the query heads of a few slices,
seed 0).  It calls only the oracle and the input generator, and writes
tests/golden/planted_peak.json; workloads/configs.py carries the same numbers
(tests/test_workloads.py checks that they agree).

Usage: python tests/golden/calibrate_peak.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import get_config, generate_all  # noqa: E402

TARGET = 0.90
SLICES = [(0, 0), (0, 3), (0, 6)]


def planted_mass(cfg, peak: float) -> float:
    cfg = cfg.with_(peak=peak)
    masses = []
    for (b, h) in SLICES:
        K, V, Q, planted, _, _ = generate_all(cfg, slices=[(b, h)])
        G = cfg.gqa
        q = Q[b:b + 1, h * G:(h + 1) * G]
        k = K[b:b + 1, h:h + 1].astype(np.float64)
        v = V[b:b + 1, h:h + 1].astype(np.float64)
        p, _, _ = oracle.attention_probs(q, k, v, sm_scale=cfg.sm_scale)
        masses.append(p[0, :, 1][:, planted[b, h]].sum(-1).mean())
    return float(np.mean(masses))


def calibrate(name: str) -> float:
    cfg = get_config(name)
    lo, hi = 0.0, 40.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if planted_mass(cfg, mid) < TARGET:
            lo = mid
        else:
            hi = mid
    return round(hi, 2)


def main():
    out = {"target_mass": TARGET, "seed": 0, "slices": SLICES,
           "cite": "SpeCache summary (papercache.org), section 2 'attention sparsity' with Figure 2 "
                   "(left): 0.5% of keys cover 90% of the attention"}
    for name in ("llama8k", "mistral32k"):
        peak = calibrate(name)
        out[name] = {"peak": peak, "mass": planted_mass(get_config(name), peak)}
        print(name, out[name], flush=True)
    out["layers32"] = out["mistral32k"]
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "planted_peak.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
