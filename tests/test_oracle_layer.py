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


# ---------------------------------------------------------------- weighted sum, top_k >= 2
# A layer whose routing weights and expert outputs are known in closed form, so
# the weighted sum of moe_weighted_sum_blend_prefill (forward_token_major.rs:
# out = sum_j w[r, j] * y[r, j] + gate * shared) is checked with weights other
# than 1 and with distinct weights inside a row.
#
# Row r's input is bf16 1.0 at column r and zero elsewhere, and router row e is
# zero except at columns 0 and 1, so the logits are exactly L[r, e] = W[e, r].
# Logits of +100, 0 and -100 give sigmoid scores of exactly 1 and 0.5 in
# float64 (exp(-100) is below half an ulp of 1) and a score below 1e-43; the
# small distinct biases order equal scores.  With renormalisation the weights
# are s_j / sum(s) * routed_scaling_factor:
#   row 0 selects experts 6, 5 (score 1) and 2 (score 0.5): w = 1, 1, 0.5
#   row 1 selects expert 0 (score 1), then 4 and 3 (score 0.5): w = 1.25, 0.625, 0.625
# Every expert has all-ones codes and block scales 1.0 with its own power-of-two
# scale2 c_e, so for a one-hot input g = v = c_e and y_e = I * c_e * fp32(silu(c_e) * c_e)
# in every column (the all-ones closed form of the FFN).  A zero gate vector gives
# gamma = 0.5; the shared expert is all ones with scale2 1.
_WS_C = [1.0, 2.0, 4.0, 0.5, 0.25, 8.0, 0.125, 16.0]
_WS_L = [[-100.0, -100.0, 0.0, -100.0, -100.0, 100.0, 100.0, -100.0],
         [100.0, -100.0, -100.0, 0.0, 0.0, -100.0, -100.0, -100.0]]
_WS_IDS = [[6, 5, 2], [0, 4, 3]]
_WS_W = [[1.0, 1.0, 0.5], [1.25, 0.625, 0.625]]


def _weighted_sum_layer():
    h, E, k, I = 64, 8, 3, 32
    s = synth.MoeShape("wsum", h, E, k, I, I, 2, synth.ROUTE_SIGMOID_BIAS, True, 2.5)

    def ones(n, kk, scale2):
        return synth.Nvfp4Tensor(n, kk, np.full((n, kk // 2), 0x22, np.uint8),
                                 np.full((n, kk // 16), 0x38, np.uint8), scale2)

    router = np.zeros((E, h), np.float32)
    router[:, 0], router[:, 1] = _WS_L[0], _WS_L[1]
    bias = (0.01 * np.arange(E) - 0.04).astype(np.float32)
    w = synth.MoeLayerWeights(shape=s, router_w=router, bias=bias, shared_gate_vec=np.zeros(h, np.float32),
                              shared=(ones(I, h, 1.0), ones(I, h, 1.0), ones(h, I, 1.0)))
    w._experts = {(e, p): ones(I, h, _WS_C[e]) if p < 2 else ones(h, I, _WS_C[e])
                  for e in range(E) for p in range(3)}
    w.lazy = False
    x = np.zeros((2, h), np.uint16)
    x[0, 0] = x[1, 1] = 0x3F80  # bf16 1.0
    return s, w, x


def _all_ones_y(c, inter):
    a = float(np.float32(c / (1.0 + math.exp(-c)) * c))
    return inter * c * a  # exact: I and c are powers of two


def test_weighted_sum_closed_form_top_k_3():
    s, w, x = _weighted_sum_layer()
    o = moe_layer_from(w, x)
    assert o["ids"].tolist() == _WS_IDS
    assert o["weights"].tolist() == _WS_W
    assert np.all(o["gamma"] == 0.5)
    shared = _all_ones_y(1.0, s.shared_inter)
    for r in range(2):
        # every term is an fp32 value times a short dyadic weight, and their
        # exponents span far less than float64's 53 bits: the sum is exact
        total = sum(_WS_W[r][j] * _all_ones_y(_WS_C[_WS_IDS[r][j]], s.moe_inter) for j in range(s.top_k))
        total += 0.5 * shared
        want = f32_to_bf16_bits(np.full(s.hidden, total, np.float64).astype(np.float32))
        assert np.array_equal(o["out"][r], want), (r, bf16_to_f64(o["out"][r][:1]), total)
