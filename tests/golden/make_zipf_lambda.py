"""Calibrate the selection-bias strength that gives the skewed workloads their Zipf expert popularity.

The skew enters through the layer's own selection-only bias: b_e = -lam * s * ln(rank_e), ranks a
seeded permutation of the experts (synth.zipf_bias).  lam is bisected so that the realised
rank-frequency curve of the routed experts has log-log slope -s (least-squares fit over the experts
that were picked at least once), with the routing computed by the oracle only.  Writes
zipf_lambda.json next to this script: lam, the slope reached, and the histogram (counts by rank).

Run from the repository root:  python tests/golden/make_zipf_lambda.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

TOKENS = {"stack": 2000, "prefill": 512}


def slope(counts: np.ndarray) -> float:
    c = np.sort(counts)[::-1].astype(np.float64)
    c = c[c > 0]
    r = np.arange(1, c.size + 1, dtype=np.float64)
    return float(np.polyfit(np.log(r), np.log(c), 1)[0])


def histogram(shape, x, gate_w, lam):
    bias = synth.zipf_bias(shape, lam)
    ids, _, _, _ = oracle.route(x, gate_w, shape.top_k, shape.routed_scale, bias)
    return np.bincount(ids.reshape(-1), minlength=shape.n_experts)


def calibrate(name):
    shape = synth.WORKLOADS[name]
    x = synth.tokens(shape, TOKENS[name], first=100000)
    gate_w = synth.gate_weights(shape)
    lo, hi = 0.0, 2.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if slope(histogram(shape, x, gate_w, mid)) > -shape.zipf_s:
            lo = mid
        else:
            hi = mid
    lam = 0.5 * (lo + hi)
    h = histogram(shape, x, gate_w, lam)
    return {"lam": lam, "s": shape.zipf_s, "slope": slope(h), "tokens": TOKENS[name],
            "counts_by_rank": sorted(h.tolist(), reverse=True)}


def main():
    oracle.build()
    out = {name: calibrate(name) for name in TOKENS}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_lambda.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    for name, r in out.items():
        print(name, "lam", r["lam"], "slope", r["slope"], "max", r["counts_by_rank"][0],
              "min", r["counts_by_rank"][-1])


if __name__ == "__main__":
    main()
