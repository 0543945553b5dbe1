"""Router logits and top-k routing (float64 arithmetic, fp32 decisions).

Follows ``forward_token_major.rs`` (``MoeLayer::forward_token_major_decode``):
a batched router GEMM over the rows produces ``gate_logits`` [n, E]; then
either ``moe_topk_sigmoid_batched`` (when a correction bias is present; it
receives the bias, ``norm_topk_prob`` and ``routed_scaling_factor``) or
``moe_topk_softmax_batched`` (receives ``norm_topk_prob`` only) writes the
top-k ids followed by the top-k weights.  ``forward_ep.rs`` shows the one-row
form (router GEMV then ``moe_topk_softmax``).

Readings where the pages are silent (each is listed in the design notes):
* the router input is the layer input itself (``router_input`` unexplained);
* the router weight is dense fp32 [E, h] (the configs' router), or NVFP4 like
  the experts (the pages' other router form);
* softmax selects on the logits (monotone in the probabilities);
* sigmoid routing adds the bias to the sigmoid score for selection only, the
  weights use the unbiased score, the optional renormalisation comes first and
  ``routed_scaling_factor`` multiplies after it in both cases;
* softmax routing takes no scaling factor (the softmax call has none);
* within a row the k ids are ordered by descending key, equal keys by
  ascending expert id;
* selection compares fp32 keys: logits rounded once to fp32 from an exact
  (float64) dot product; sigmoid keys are fp32(fp32(s) + bias).

Pinned by tests/test_oracle_route.py: brute-force exact dot products
(math.fsum) for the logits; numpy's stable argsort for the selection order
including ties; closed forms for a zero router; sums of renormalised weights;
the k-th/(k+1)-th key margin against constructed keys and a brute force over
every k-subset.
"""

from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .formats import bf16_to_f64, dequant_nvfp4, f64_to_f32

ROUTE_SOFTMAX = 0
ROUTE_SIGMOID_BIAS = 1


def router_logits(x_bits: np.ndarray, router_w) -> np.ndarray:
    """L[r, e] = fp32(sum_t x[r, t] * W[e, t]); bf16*fp32 products are exact in float64.

    ``router_w`` is a dense fp32 [E, h] array, or an NVFP4 matrix [E, h]
    (an object with n, k, packed, scales, scale2): the gate projection is then
    an NVFP4 GEMV/GEMM like the experts' (``forward_ep.rs`` calls
    ``w4a16_decode_gemv``, ``forward_token_major.rs`` ``w4a16_gemm``, on the
    router input).  Its weights are decoded exactly in float64 first."""
    x = bf16_to_f64(x_bits)
    if hasattr(router_w, "packed"):
        w = dequant_nvfp4(router_w.packed, router_w.scales, router_w.scale2, router_w.n, router_w.k)
    else:
        w = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    return f64_to_f32(x @ w.T)


def shared_gate(x_bits: np.ndarray, gate_vec) -> np.ndarray:
    """gamma[r] = sigmoid(x_r . g_s) in float64: the shared expert's blend gate.

    Without a gate vector (``None``) the shared expert is added ungated,
    gamma = 1: ``forward_token_major.rs`` calls ``residual_add`` instead of
    ``moe_batched_blend`` when ``shared_expert_gate.weight`` is null."""
    x = bf16_to_f64(x_bits)
    if gate_vec is None:
        return np.ones(x.shape[0], dtype=np.float64)
    z = x @ np.asarray(gate_vec, dtype=np.float32).astype(np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def select_topk(keys32: np.ndarray, k: int) -> List[int]:
    """The k largest fp32 keys of one row: descending key, ties by lower id."""
    keys = [float(v) for v in np.asarray(keys32, dtype=np.float32)]
    order = sorted(range(len(keys)), key=lambda e: (-keys[e], e))
    return order[:k]


def topk_softmax(logits32: np.ndarray, k: int, norm_topk_prob: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax routing of each row: ids int32 [R, k], weights fp32 [R, k]."""
    R, E = logits32.shape
    ids = np.zeros((R, k), dtype=np.int32)
    wts = np.zeros((R, k), dtype=np.float32)
    for r in range(R):
        sel = select_topk(logits32[r], k)
        L = logits32[r].astype(np.float64)
        p = np.exp(L - L.max())
        p = p / p.sum()
        w = p[sel]
        if norm_topk_prob:
            w = w / w.sum()
        ids[r] = sel
        wts[r] = f64_to_f32(w)
    return ids, wts


def sigmoid_scores(logits32: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-L)) in float64."""
    return 1.0 / (1.0 + np.exp(-np.asarray(logits32, dtype=np.float64)))


def sigmoid_keys(logits32: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Selection keys fp32(fp32(s) + bias); an fp32 add is the fp32 rounding of the exact sum."""
    s32 = f64_to_f32(sigmoid_scores(logits32)).astype(np.float64)
    return f64_to_f32(s32 + np.asarray(bias, dtype=np.float32).astype(np.float64))


def topk_sigmoid_bias(logits32: np.ndarray, bias: np.ndarray, k: int, norm_topk_prob: bool,
                      routed_scaling_factor: float) -> Tuple[np.ndarray, np.ndarray]:
    """Sigmoid + correction-bias routing of each row: ids int32 [R, k], weights fp32 [R, k]."""
    R, E = logits32.shape
    ids = np.zeros((R, k), dtype=np.int32)
    wts = np.zeros((R, k), dtype=np.float32)
    s = sigmoid_scores(logits32)
    keys = sigmoid_keys(logits32, bias)
    for r in range(R):
        sel = select_topk(keys[r], k)
        w = s[r][sel]
        if norm_topk_prob:
            w = w / w.sum()
        w = w * float(np.float32(routed_scaling_factor))
        ids[r] = sel
        wts[r] = f64_to_f32(w)
    return ids, wts


def route(x_bits, router_w, bias, route_kind: int, k: int, norm_topk_prob: bool,
          routed_scaling_factor: float):
    """Logits, ids and weights for all rows of ``x_bits``."""
    L = router_logits(x_bits, router_w)
    if route_kind == ROUTE_SOFTMAX:
        ids, w = topk_softmax(L, k, norm_topk_prob)
    elif route_kind == ROUTE_SIGMOID_BIAS:
        ids, w = topk_sigmoid_bias(L, bias, k, norm_topk_prob, routed_scaling_factor)
    else:
        raise ValueError(f"unknown route kind {route_kind}")
    return L, ids, w


def selection_keys(logits32: np.ndarray, bias, route_kind: int) -> np.ndarray:
    """The fp32 keys top-k compares: the logits for softmax routing, fp32(fp32(s) + bias)
    for sigmoid routing."""
    if route_kind == ROUTE_SOFTMAX:
        return np.asarray(logits32, dtype=np.float32)
    if route_kind == ROUTE_SIGMOID_BIAS:
        return sigmoid_keys(logits32, bias)
    raise ValueError(f"unknown route kind {route_kind}")


def topk_margin(keys32: np.ndarray, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest key of a row (inf if k == E).

    The selection is unique when the gap is positive; a gap below the rounding
    noise of an independent evaluation of the logits marks a near-tie, where two
    correct implementations may pick different experts."""
    v = np.sort(np.asarray(keys32, dtype=np.float64))[::-1]
    if k >= len(v):
        return math.inf
    return float(v[k - 1] - v[k])
