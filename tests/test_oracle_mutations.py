"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case patches one plausible error into the oracle (swapped nibbles, an
exponent bias off by one, silu on the wrong projection, a dropped shared
term, ties broken the wrong way, a sorted union, renormalising over all
experts, biased sigmoid weights, a local union without its range filter, a
rank's partial that keeps remote slots, an ungated shared expert dropped, a
weighted sum that ignores the routing weights or pairs them with the wrong
slots, a near-tie margin taken between the wrong ranks) and runs the pin that
should catch it.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import ffn as FF
from oracle import layer as LY
from oracle import route as RT
from oracle import union as UN

import test_oracle_ffn as T_ffn
import test_oracle_formats as T_fmt
import test_oracle_layer as T_layer
import test_oracle_route as T_route
import test_oracle_union as T_union


def _swapped_unpack(packed, n, k):
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2] = p >> 4
    codes[:, 1::2] = p & 0x0F
    return codes


def _bad_e4m3_table():
    t = F.E4M3FN_TABLE.copy()
    fin = np.isfinite(t)
    t[fin] = t[fin] * 2.0  # exponent bias 6 instead of 7
    return t


def _silu_on_up(w_gate, w_up, w_down, x64):
    x64 = np.atleast_2d(x64)
    g = F.f64_to_f32(x64 @ w_gate.T).astype(np.float64)
    v = F.f64_to_f32(x64 @ w_up.T).astype(np.float64)
    a = F.f64_to_f32(FF.silu(v) * g).astype(np.float64)
    return F.f64_to_f32(a @ w_down.T)


def _ties_to_higher(keys32, k):
    keys = [float(v) for v in np.asarray(keys32, dtype=np.float32)]
    return sorted(range(len(keys)), key=lambda e: (-keys[e], -e))[:k]


def _sorted_union(ids):
    u, U, s2u, m = UN.expert_union.__wrapped__(ids)
    order = np.argsort(u, kind="stable")
    return u[order], U, np.argsort(order)[s2u], m[order]


def _norm_over_all(logits32, k, norm):
    R, E = logits32.shape
    ids = np.zeros((R, k), np.int32)
    w = np.zeros((R, k), np.float32)
    for r in range(R):
        sel = RT.select_topk(logits32[r], k)
        L = logits32[r].astype(np.float64)
        p = np.exp(L - L.max())
        p /= p.sum()
        ids[r], w[r] = sel, p[sel].astype(np.float32)
    return ids, w


def _biased_weights(logits32, bias, k, norm, rsf):
    keys = RT.sigmoid_keys(logits32, bias).astype(np.float64)
    R = logits32.shape[0]
    ids = np.zeros((R, k), np.int32)
    w = np.zeros((R, k), np.float32)
    for r in range(R):
        sel = RT.select_topk(keys[r], k)
        ww = keys[r][sel]
        if norm:
            ww = ww / ww.sum()
        ids[r], w[r] = sel, (ww * rsf).astype(np.float32)
    return ids, w


def test_swapped_nibbles_caught(monkeypatch):
    monkeypatch.setattr(F, "unpack_e2m1_codes", _swapped_unpack)
    with pytest.raises(AssertionError):
        T_fmt.test_nvfp4_layout_golden()


def test_bad_exponent_bias_caught(monkeypatch):
    monkeypatch.setattr(F, "E4M3FN_TABLE", _bad_e4m3_table())
    with pytest.raises(AssertionError):
        T_fmt.test_e4m3fn_all_bytes_match_torch()


def test_silu_on_wrong_projection_caught(monkeypatch):
    monkeypatch.setattr(FF, "ffn_dense", _silu_on_up)
    with pytest.raises(AssertionError):
        T_ffn.test_one_hot_closed_form()


def test_dropped_shared_term_caught(monkeypatch):
    def no_shared(w_row, y_row, gamma, shared_row):
        acc = sum(float(w_row[j]) * y_row[j].astype(np.float64) for j in range(len(w_row)))
        return F.f32_to_bf16_bits(F.f64_to_f32(acc))
    monkeypatch.setattr(LY, "blend_row", no_shared)
    with pytest.raises(AssertionError):
        T_layer.test_single_expert_output_closed_form()


def test_ties_to_higher_id_caught(monkeypatch):
    monkeypatch.setattr(RT, "select_topk", _ties_to_higher)
    with pytest.raises(AssertionError):
        T_route.test_select_matches_stable_argsort_with_ties()


def test_sorted_union_caught(monkeypatch):
    import functools
    real = UN.expert_union
    wrapped = functools.wraps(real)(lambda ids: real(ids))
    monkeypatch.setattr(UN, "expert_union", wrapped)
    monkeypatch.setattr(T_union, "expert_union", _sorted_union)
    with pytest.raises(AssertionError):
        T_union.test_union_exhaustive_tiny()


def test_renormalise_over_all_experts_caught(monkeypatch):
    monkeypatch.setattr(RT, "topk_softmax", _norm_over_all)
    with pytest.raises(AssertionError):
        T_route.test_softmax_norm_is_softmax_over_selected()


def test_biased_sigmoid_weights_caught(monkeypatch):
    monkeypatch.setattr(RT, "topk_sigmoid_bias", _biased_weights)
    with pytest.raises(AssertionError):
        T_route.test_sigmoid_weights_are_unbiased_scores()


def _local_union_keeps_remote(ids, lo, hi):
    # the mistake: the range filter is dropped, every selected id stays local
    return UN.expert_union(ids)


def test_local_union_without_range_filter_caught(monkeypatch):
    monkeypatch.setattr(T_union, "expert_union_local", _local_union_keeps_remote)
    with pytest.raises(AssertionError):
        T_union.test_local_union_exhaustive_tiny()


def test_partial_with_remote_slots_caught(monkeypatch):
    real = LY.routed_partial_row
    # the mistake: every slot counts as local
    monkeypatch.setattr(LY, "routed_partial_row", lambda w_row, y_row, local: real(w_row, y_row, np.ones_like(local)))
    with pytest.raises(AssertionError):
        T_layer.test_ep_partial_single_expert_closed_form()


def test_ungated_shared_as_zero_caught(monkeypatch):
    real = RT.shared_gate

    def zero_when_ungated(x_bits, gate_vec):
        if gate_vec is None:
            return np.zeros(np.atleast_2d(x_bits).shape[0])
        return real(x_bits, gate_vec)
    monkeypatch.setattr(LY, "shared_gate", zero_when_ungated)
    with pytest.raises(AssertionError):
        T_layer.test_ungated_shared_expert_is_gate_one()


def test_weights_ignored_caught(monkeypatch):
    real = LY.blend_row
    # the mistake: every routed expert enters the sum with weight 1
    monkeypatch.setattr(LY, "blend_row", lambda w_row, y_row, gamma, shared_row: real(
        np.ones_like(w_row), y_row, gamma, shared_row))
    with pytest.raises(AssertionError):
        T_layer.test_weighted_sum_closed_form_top_k_3()


def test_weights_paired_with_reversed_slots_caught(monkeypatch):
    real = LY.blend_row
    # the mistake: weight j multiplies the output of slot k - 1 - j
    monkeypatch.setattr(LY, "blend_row", lambda w_row, y_row, gamma, shared_row: real(
        w_row[::-1], y_row, gamma, shared_row))
    with pytest.raises(AssertionError):
        T_layer.test_weighted_sum_closed_form_top_k_3()


def test_margin_between_wrong_ranks_caught(monkeypatch):
    def off_by_one(keys32, k):
        v = np.sort(np.asarray(keys32, dtype=np.float64))[::-1]
        # the mistake: ranks k+1 and k+2 instead of k and k+1
        return float(v[k] - v[k + 1]) if k + 1 < len(v) else float("inf")
    monkeypatch.setattr(RT, "topk_margin", off_by_one)
    with pytest.raises(AssertionError):
        T_route.test_topk_margin_constructed_keys()
