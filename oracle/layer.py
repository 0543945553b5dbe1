"""The whole routed-MoE layer for a verify's rows, as a plain definition.

Steps, in the order of ``MoeLayer::forward_token_major_decode``
(``forward_token_major.rs``): router logits, batched top-k, gate+up,
silu+down, weighted sum plus the blend of the gated shared expert into the
output.  Single GPU, so ``out`` holds the full sum ("Function forward_moe"
rustdoc, summary: the output is partial only when experts or the shared
expert are split across ranks).

For each row r (independently of every other row):

    out[r] = bf16(fp32( sum_{j<k} w[r, j] * FFN_{id[r, j]}(x_r) + gamma_r * FFN_shared(x_r) ))

with the j-sum in float64 in ascending j, gamma_r = sigmoid(x_r . g_s)
(the shared-expert gate is a sigmoid of a dot with a gate vector: the
``moe_weighted_sum_blend_prefill`` call receives the input and
``shared_expert_gate.weight``), and FFN as in ``oracle.ffn``.

Because every row is computed alone, deduplicating experts across rows cannot
change any row's result ("Function forward_moe" rustdoc, "RETRACTED
(2026-08-29)" note: the same output bytes with or without the union).  The loop below
groups (row, expert) pairs by expert only so an expert is decoded once; each
pair's value is the same as if computed alone.
"""

from __future__ import annotations

from typing import Callable, Dict, Iterable, Optional, Sequence

import numpy as np

from .formats import bf16_to_f64, f32_to_bf16_bits, f64_to_f32
from .ffn import dequant, ffn_dense
from .route import route, shared_gate
from .union import expert_union, expert_union_local


def blend_row(w_row: np.ndarray, y_row: np.ndarray, gamma: float, shared_row: np.ndarray) -> np.ndarray:
    """bf16(fp32(sum_j w[j] * y[j] + gamma * shared)), the j-sum in float64 in ascending j.

    Pinned with routing weights other than 1 (and distinct within a row) by a
    closed-form layer in tests/test_oracle_layer.py."""
    acc = np.zeros(y_row.shape[-1], dtype=np.float64)
    for j in range(len(w_row)):
        acc = acc + float(w_row[j]) * y_row[j].astype(np.float64)
    acc = acc + float(gamma) * shared_row.astype(np.float64)
    return f32_to_bf16_bits(f64_to_f32(acc))


def routed_partial_row(w_row: np.ndarray, y_row: np.ndarray, local: np.ndarray) -> np.ndarray:
    """fp32(sum_j w[j] * y[j]) over the slots j with ``local[j]``, in float64 in
    ascending j (zero when no slot is local): one rank's share of the routed
    sum before the all-reduce (``forward_token_major.rs`` under EP blends with a
    zeroed shared term, then all-reduces the output)."""
    acc = np.zeros(y_row.shape[-1], dtype=np.float64)
    for j in range(len(w_row)):
        if local[j]:
            acc = acc + float(w_row[j]) * y_row[j].astype(np.float64)
    return f64_to_f32(acc)


def ep_combine(reduced: np.ndarray, gamma: np.ndarray, shared_y: np.ndarray) -> np.ndarray:
    """out[r] = bf16(fp32(reduced[r] + gamma[r] * shared[r])): the shared expert
    added after the all-reduce (``forward_token_major.rs``: ``moe_batched_blend``,
    or ``residual_add`` with gamma = 1 when the gate weight is null)."""
    red = np.asarray(reduced, dtype=np.float32).astype(np.float64)
    s = np.asarray(shared_y, dtype=np.float32).astype(np.float64)
    g = np.asarray(gamma, dtype=np.float64)[:, None]
    return f32_to_bf16_bits(f64_to_f32(red + g * s))


def moe_layer(x_bits: np.ndarray, *, router_w: np.ndarray, bias: Optional[np.ndarray],
              shared_gate_vec: Optional[np.ndarray], shared: Sequence, expert: Callable[[int, int], object],
              route_kind: int, top_k: int, norm_topk_prob: bool, routed_scaling_factor: float,
              rows: Optional[Iterable[int]] = None,
              expert_range: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Evaluate the layer on bf16 rows ``x_bits`` [R, h].

    ``shared`` is (gate, up, down) NVFP4 matrices; ``expert(e, p)`` returns
    routed expert e's projection p (0 gate, 1 up, 2 down).  ``rows`` limits
    the expert FFNs and the output to a subset of rows (routing and the union
    are always computed for all rows).  Returns a dict with ``logits``,
    ``ids``, ``weights``, ``gamma``, ``union_ids``, ``union_count``,
    ``slot_to_union``, ``row_mask``, ``y`` (fp32 [R, k, h]; NaN for rows not
    evaluated), ``shared_y`` (fp32 [R, h]) and ``out`` (bf16 bits [R, h];
    0 for rows not evaluated).

    ``shared_gate_vec`` None adds the shared expert ungated (gamma = 1).
    With ``expert_range`` = (lo, hi) the result also holds one rank's share:
    ``local_union_ids``, ``local_union_count``, ``local_slot_to_union``,
    ``local_row_mask`` (``expert_union_local``) and ``partial`` (fp32 [R, h],
    the routed sum over the row's slots whose expert lies in [lo, hi); NaN for
    rows not evaluated).
    """
    x_bits = np.atleast_2d(np.asarray(x_bits, dtype=np.uint16))
    R, h = x_bits.shape
    k = top_k
    logits, ids, w = route(x_bits, router_w, bias, route_kind, k, norm_topk_prob, routed_scaling_factor)
    union_ids, U, slot_to_union, row_mask = expert_union(ids)
    gamma = shared_gate(x_bits, shared_gate_vec)
    rows = list(range(R)) if rows is None else sorted(set(int(r) for r in rows))
    x64 = bf16_to_f64(x_bits)

    y = np.full((R, k, h), np.nan, dtype=np.float32)
    # Group the (row, slot) pairs of the evaluated rows by expert.
    pairs: Dict[int, list] = {}
    for r in rows:
        for j in range(k):
            pairs.setdefault(int(ids[r, j]), []).append((r, j))
    for e, plist in pairs.items():
        wg, wu, wd = (dequant(expert(e, p)) for p in range(3))
        for (r, j) in plist:
            y[r, j] = ffn_dense(wg, wu, wd, x64[r:r + 1])[0]

    shared_y = np.full((R, h), np.nan, dtype=np.float32)
    sg, su, sd = (dequant(t) for t in shared)
    for r in rows:
        shared_y[r] = ffn_dense(sg, su, sd, x64[r:r + 1])[0]

    out = np.zeros((R, h), dtype=np.uint16)
    for r in rows:
        out[r] = blend_row(w[r], y[r], gamma[r], shared_y[r])

    res = dict(logits=logits, ids=ids, weights=w, gamma=gamma, union_ids=union_ids,
               union_count=U, slot_to_union=slot_to_union, row_mask=row_mask,
               y=y, shared_y=shared_y, out=out, rows=np.array(rows, dtype=np.int32))
    if expert_range is not None:
        lo, hi = int(expert_range[0]), int(expert_range[1])
        lu, lU, ls2u, lmask = expert_union_local(ids, lo, hi)
        partial = np.full((R, h), np.nan, dtype=np.float32)
        for r in rows:
            partial[r] = routed_partial_row(w[r], y[r], (ids[r] >= lo) & (ids[r] < hi))
        res.update(local_union_ids=lu, local_union_count=lU, local_slot_to_union=ls2u, local_row_mask=lmask,
                   partial=partial)
    return res


def moe_layer_from(weights, x_bits: np.ndarray, rows: Optional[Iterable[int]] = None,
                   expert_range: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Convenience wrapper: ``weights`` has router_w, bias, shared_gate_vec, shared,
    expert(e, p) and a ``shape`` with the routing parameters."""
    s = weights.shape
    return moe_layer(x_bits, router_w=weights.router_w, bias=weights.bias,
                     shared_gate_vec=weights.shared_gate_vec, shared=weights.shared,
                     expert=weights.expert, route_kind=s.route_kind, top_k=s.top_k,
                     norm_topk_prob=s.norm_topk_prob, routed_scaling_factor=s.routed_scaling_factor,
                     rows=rows, expert_range=expert_range)
