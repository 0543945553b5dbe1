"""The expert feed-forward: gate+up, silu(gate)*up, down (float64 sums).

``forward_token_major.rs`` runs ``moe_expert_gate_up_shared_prefill`` (the
gate and up projections of each selected expert, plus the shared expert's)
and then ``moe_expert_silu_down_shared_prefill`` (silu of the gate times the
up projection, then the down projection; the same for the shared expert).
"Function forward_moe" rustdoc, SHARED-expert note: the shared expert uses the
same weights for every row and runs over all rows.

For one activation row x (h values) and one expert with NVFP4 projections
gate [I, h], up [I, h], down [h, I]:

    g = fp32(W_gate @ x),  v = fp32(W_up @ x)      (float64 sums)
    a = fp32(silu(g) * v),  silu(z) = z / (1 + exp(-z))
    y = fp32(W_down @ a)                          (float64 sum)

Pinned by tests/test_oracle_ffn.py: closed forms (all-ones weights; one-hot
weights selecting entries of x) and brute-force math.fsum dot products on a
small random expert.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .formats import dequant_nvfp4, f64_to_f32


def dequant(t) -> np.ndarray:
    """Any object with n, k, packed, scales, scale2 (an NVFP4 matrix) -> float64 [n, k]."""
    return dequant_nvfp4(t.packed, t.scales, t.scale2, t.n, t.k)


def silu(z: np.ndarray) -> np.ndarray:
    """z / (1 + exp(-z)); for z far below zero exp(-z) overflows to inf and the
    quotient is the limit -0.0 (the overflow warning is silenced, not the value)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def ffn_dense(w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """FFN of rows x64 [m, h] with dequantised float64 weights -> y fp32 [m, h]."""
    x64 = np.atleast_2d(np.asarray(x64, dtype=np.float64))
    g = f64_to_f32(x64 @ w_gate.T).astype(np.float64)
    v = f64_to_f32(x64 @ w_up.T).astype(np.float64)
    a = f64_to_f32(silu(g) * v).astype(np.float64)
    return f64_to_f32(a @ w_down.T)


def ffn_nvfp4(gate, up, down, x64: np.ndarray) -> np.ndarray:
    """FFN of rows x64 [m, h] with NVFP4 projections (objects as in ``dequant``)."""
    return ffn_dense(dequant(gate), dequant(up), dequant(down), x64)
