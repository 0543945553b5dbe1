"""Tune the row correlation of the 256-expert K=4 verify workload.

The "Function forward_moe" rustdoc ("amortize PARTIALLY" note) reports a mean
union of 23.35 selected experts over K = 4 consecutive tokens.  The synthetic
workload mixes each verify row with row 0 (x_r = a*x_0 + sqrt(1-a^2)*z_r); this
script evaluates the oracle's routing over steps 0..999 for a grid of ``a``
and prints the mean union size, from which ``synth.C3_ROW_CORR`` was chosen.

Run: python tests/golden/tune_c3_row_corr.py
"""

import dataclasses
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import synth  # noqa: E402
from oracle.route import route  # noqa: E402
from oracle.union import expert_union  # noqa: E402


def mean_union(shape, steps=1000):
    w = synth.router_weight(shape)
    b = synth.correction_bias(shape)
    us = []
    for s in range(steps):
        x = synth.activations(shape, s)
        _, ids, _ = route(x, w, b, shape.route_kind, shape.top_k, shape.norm_topk_prob,
                          shape.routed_scaling_factor)
        us.append(expert_union(ids)[1])
    return float(np.mean(us)), float(np.std(us))


if __name__ == "__main__":
    base = synth.CONFIGS["c3_e256_verify4"]
    grid = [float(a) for a in sys.argv[1:]] or [0.55, 0.58, 0.60, 0.61, 0.62, 0.65]
    for a in grid:
        m, sd = mean_union(dataclasses.replace(base, row_corr=a))
        print(f"a={a:.3f} mean_U={m:.3f} std={sd:.2f}", flush=True)
