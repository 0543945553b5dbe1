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


def test_ungated_shared_expert_is_gate_one():
    # A gate vector with x . g = 100 gives sigmoid = 1 exactly in float64
    # (exp(-100) is below half an ulp of 1), so the gated layer must equal the
    # ungated one (gamma = 1) bit for bit.
    s, w = _tiny(rows=1)
    x = synth.activations(s, 5)
    xf = bf16_to_f64(x)[0]
    w.shared_gate_vec = (100.0 * xf / np.dot(xf, xf)).astype(np.float32)
    gated = moe_layer_from(w, x)
    assert np.all(gated["gamma"] == 1.0)
    w.shared_gate_vec = None
    ungated = moe_layer_from(w, x)
    assert np.all(ungated["gamma"] == 1.0)
    assert np.array_equal(gated["out"], ungated["out"])


def test_ep_partial_single_expert_closed_form():
    # k = 1 with renormalisation: each row's partial is its expert's y when
    # the expert is local, else exactly zero.
    s, w = _tiny(top_k=1, rows=3)
    x = synth.activations(s, 6)
    for lo, hi in [(0, 4), (4, 8), (0, 8), (3, 3)]:
        o = moe_layer_from(w, x, expert_range=(lo, hi))
        for r in range(s.rows):
            e = int(o["ids"][r, 0])
            want = o["y"][r, 0] if lo <= e < hi else np.zeros(s.hidden, np.float32)
            assert np.array_equal(o["partial"][r], want)


def test_ep_partials_reduce_to_the_layer():
    # The ranks' partials add up to the routed sum, and the combine of their
    # sum with the shared expert is the layer's output to within one bf16
    # rounding (the reduced sum is rounded to fp32 once more before the add).
    from oracle.layer import ep_combine
    s, w = _tiny(route_kind=synth.ROUTE_SIGMOID_BIAS, top_k=3, rows=4)
    x = synth.activations(s, 7)
    full = moe_layer_from(w, x)
    ranges = [(0, 2), (2, 5), (5, 8)]
    parts = [moe_layer_from(w, x, expert_range=rg) for rg in ranges]
    assert sum(p["local_union_count"] for p in parts) == full["union_count"]
    red = np.sum([p["partial"].astype(np.float64) for p in parts], axis=0)
    for r in range(s.rows):
        routed = sum(float(full["weights"][r, j]) * full["y"][r, j].astype(np.float64) for j in range(s.top_k))
        mag = sum(abs(float(full["weights"][r, j])) * np.abs(full["y"][r, j].astype(np.float64))
                  for j in range(s.top_k))
        assert np.all(np.abs(red[r] - routed) <= 4 * 2.0 ** -24 * mag)
    out = ep_combine(red.astype(np.float32), full["gamma"], full["shared_y"])
    g, ref = bf16_to_f64(out), bf16_to_f64(full["out"])
    assert np.all(np.abs(g - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)
