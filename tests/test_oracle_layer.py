"""Pins for the oracle's whole-layer definition (CPU only)."""

import math

import numpy as np
import pytest

import synth
from oracle.formats import bf16_to_f64, f32_to_bf16_bits
from oracle.layer import moe_layer, moe_layer_from
from oracle import ffn as FF


def _tiny(route_kind=synth.ROUTE_SOFTMAX, top_k=4, rows=3, gate_zero=False):
    s = synth.MoeShape("t", 64, 8, top_k, 32, 32, rows, route_kind, True, 2.5 if route_kind else 1.0)
    w = synth.layer_weights(s)
    if gate_zero:
        w.shared_gate_vec = np.zeros_like(w.shared_gate_vec)
    return s, w


def test_zero_shared_gate_is_half():
    s, w = _tiny(gate_zero=True)
    o = moe_layer_from(w, synth.activations(s, 0))
    assert np.all(o["gamma"] == 0.5)


def test_single_expert_output_closed_form():
    # k = 1 with renormalisation: w = 1, so out = bf16(fp32(y + gamma * s)).
    s, w = _tiny(top_k=1)
    x = synth.activations(s, 3)
    o = moe_layer_from(w, x)
    assert np.all(o["weights"] == 1.0)
    xf = bf16_to_f64(x)
    for r in range(s.rows):
        e = int(o["ids"][r, 0])
        y = FF.ffn_nvfp4(*(w.expert(e, p) for p in range(3)), xf[r:r + 1])[0].astype(np.float64)
        sh = FF.ffn_nvfp4(*w.shared, xf[r:r + 1])[0].astype(np.float64)
        ref = f32_to_bf16_bits((y + o["gamma"][r] * sh).astype(np.float32))
        assert np.array_equal(o["out"][r], ref)


@pytest.mark.parametrize("kind", [synth.ROUTE_SOFTMAX, synth.ROUTE_SIGMOID_BIAS])
def test_rows_are_independent(kind):
    # Each row's output equals the one-row evaluation of that row, bit for bit.
    s, w = _tiny(route_kind=kind, rows=5)
    x = synth.activations(s, 1)
    full = moe_layer_from(w, x)
    for r in range(s.rows):
        one = moe_layer_from(w, x[r:r + 1])
        assert np.array_equal(full["out"][r], one["out"][0])
        assert np.array_equal(full["ids"][r], one["ids"][0])
        assert np.array_equal(full["weights"][r], one["weights"][0])


def test_row_subset_matches_full():
    s, w = _tiny(rows=4)
    x = synth.activations(s, 2)
    full = moe_layer_from(w, x)
    sub = moe_layer_from(w, x, rows=[1, 3])
    assert np.array_equal(sub["out"][[1, 3]], full["out"][[1, 3]])
    assert np.array_equal(sub["ids"], full["ids"])


def test_output_is_weighted_sum_plus_gated_shared():
    # out[r] = bf16(fp32(sum_j w[r, j] * y[r, j] + gamma_r * shared_y[r])), the
    # sum taken in float64 in ascending j.
    s, w = _tiny(top_k=2, rows=2)
    x = synth.activations(s, 4)
    o = moe_layer_from(w, x)
    xf = bf16_to_f64(x)
    for r in range(s.rows):
        routed = sum(float(o["weights"][r, j]) * o["y"][r, j].astype(np.float64) for j in range(2))
        total = routed + o["gamma"][r] * o["shared_y"][r].astype(np.float64)
        assert np.array_equal(o["out"][r], f32_to_bf16_bits(total.astype(np.float32)))
