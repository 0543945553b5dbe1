"""Pins for the oracle's router logits and top-k routing (CPU only)."""

import math

import numpy as np
import pytest

from oracle import route as RT
from oracle.formats import bf16_to_f64


def _bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_logits_match_exact_sums():
    rng = np.random.default_rng(11)
    R, E, h = 3, 24, 512
    x = _bf16_bits(rng.standard_normal((R, h)))
    w = (rng.standard_normal((E, h)) / math.sqrt(h)).astype(np.float32)
    L = RT.router_logits(x, w)
    xf = bf16_to_f64(x)
    mism = 0
    for r in range(R):
        for e in range(E):
            exact = math.fsum(float(a) * float(b) for a, b in zip(xf[r], w[e].astype(np.float64)))
            ref = np.float32(exact)
            if L[r, e] != ref:
                mism += 1
                assert abs(float(L[r, e]) - float(ref)) <= np.spacing(np.float32(abs(ref))), (r, e)
    assert mism <= 1


def test_logits_one_hot_input():
    E, h = 8, 64
    w = np.random.default_rng(2).standard_normal((E, h)).astype(np.float32)
    x = np.zeros((1, h), np.uint16)
    x[0, 17] = 0x3F80  # bf16 1.0
    assert np.array_equal(RT.router_logits(x, w)[0], w[:, 17])


def test_select_matches_stable_argsort_with_ties():
    rng = np.random.default_rng(12)
    for trial in range(200):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        keys = rng.integers(-3, 4, size=E).astype(np.float32)  # many exact ties
        ref = np.argsort(-keys.astype(np.float64), kind="stable")[:k].tolist()
        assert RT.select_topk(keys, k) == ref


def test_zero_router_softmax():
    E, k = 16, 4
    L = np.zeros((2, E), np.float32)
    ids, w = RT.topk_softmax(L, k, True)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(w == np.float32(0.25))
    ids, w = RT.topk_softmax(L, k, False)
    assert np.all(w == np.float32(1.0 / 16))


def test_zero_router_sigmoid_selects_by_bias():
    E, k, rsf = 32, 5, 2.5
    bias = np.random.default_rng(4).uniform(-0.1, 0.1, E).astype(np.float32)
    L = np.zeros((1, E), np.float32)
    ids, w = RT.topk_sigmoid_bias(L, bias, k, True, rsf)
    keys = (np.float32(0.5) + bias).astype(np.float32)
    assert ids[0].tolist() == np.argsort(-keys.astype(np.float64), kind="stable")[:k].tolist()
    assert np.all(w == np.float32(rsf / k))
    ids, w = RT.topk_sigmoid_bias(L, bias, k, False, rsf)
    assert np.all(w == np.float32(0.5 * rsf))


def test_topk_equals_all_experts():
    rng = np.random.default_rng(13)
    L = rng.standard_normal((3, 8)).astype(np.float32)
    ids, w = RT.topk_softmax(L, 8, True)
    for r in range(3):
        assert sorted(ids[r].tolist()) == list(range(8))
        assert abs(float(w[r].astype(np.float64).sum()) - 1.0) < 1e-6


def test_softmax_norm_is_softmax_over_selected():
    rng = np.random.default_rng(14)
    L = (rng.standard_normal((6, 64)) * 3).astype(np.float32)
    ids, w = RT.topk_softmax(L, 8, True)
    for r in range(6):
        sel = L[r, ids[r]].astype(np.float64)
        ref = np.exp(sel - sel.max())
        ref /= ref.sum()
        np.testing.assert_allclose(w[r].astype(np.float64), ref, rtol=1e-7, atol=0)
        assert np.all(np.diff(sel) <= 0)  # descending logits


def test_weights_sum_invariants():
    rng = np.random.default_rng(15)
    L = rng.standard_normal((8, 256)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 256).astype(np.float32)
    _, w = RT.topk_softmax(L, 8, True)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) < 1e-6)
    _, w = RT.topk_sigmoid_bias(L, bias, 8, True, 2.5)
    assert np.all(np.abs(w.astype(np.float64).sum(1) / 2.5 - 1.0) < 1e-6)


def test_sigmoid_weights_are_unbiased_scores():
    # Weights use sigmoid(L) without the bias: a large bias changes the
    # selection but not the weight of a selected expert.
    L = np.array([[0.0, 1.0, -1.0, 2.0]], np.float32)
    bias = np.array([5.0, 0.0, 0.0, 0.0], np.float32)
    ids, w = RT.topk_sigmoid_bias(L, bias, 2, False, 1.0)
    assert ids[0].tolist() == [0, 3]
    assert w[0, 0] == np.float32(0.5)
    assert w[0, 1] == np.float32(1.0 / (1.0 + math.exp(-2.0)))


def test_sigmoid_keys_fp32_add():
    L = np.array([[0.25, -3.0]], np.float32)
    bias = np.array([0.01, -0.02], np.float32)
    k = RT.sigmoid_keys(L, bias)
    s32 = np.float32(1.0 / (1.0 + math.exp(-0.25)))
    assert k[0, 0] == np.float32(s32 + np.float32(0.01))


# ---------------------------------------------------------------- NVFP4 router
def _nvfp4_router(E, h, scale2, seed):
    import synth
    t = synth.nvfp4_random(synth.CONFIGS["c0_tiny"], E, h, 77, seed)
    t.scale2 = scale2
    return t


def test_nvfp4_router_equals_dense_router_of_its_values():
    # With a power-of-two scale2 every decoded weight (e2m1 * e4m3 * 2^-3, at
    # most 6 significant bits) is an fp32 value, so the NVFP4 router must give
    # the dense fp32 router's logits bit for bit.  The decode is checked by
    # hand from the bit fields (low nibble = even column).
    from oracle.formats import E2M1_TABLE, E4M3FN_TABLE
    E, h = 12, 256
    t = _nvfp4_router(E, h, 0.125, 1)
    dense = np.zeros((E, h), np.float32)
    for e in range(E):
        for c in range(h):
            byte = int(t.packed[e, c // 2])
            code = (byte >> (4 * (c & 1))) & 0xF
            dense[e, c] = np.float32(E2M1_TABLE[code] * E4M3FN_TABLE[int(t.scales[e, c // 16])] * 0.125)
    x = _bf16_bits(np.random.default_rng(4).standard_normal((3, h)))
    assert np.array_equal(RT.router_logits(x, t), RT.router_logits(x, dense))


def test_nvfp4_router_logits_match_exact_sums():
    from oracle.formats import dequant_nvfp4
    E, h = 10, 512
    t = _nvfp4_router(E, h, 0.0871, 2)   # scale2 not a power of two
    x = _bf16_bits(np.random.default_rng(5).standard_normal((2, h)))
    L = RT.router_logits(x, t)
    W = dequant_nvfp4(t.packed, t.scales, t.scale2, E, h)
    xf = bf16_to_f64(x)
    for r in range(2):
        for e in range(E):
            ref = np.float32(math.fsum(float(a) * float(b) for a, b in zip(xf[r], W[e])))
            assert abs(float(L[r, e]) - float(ref)) <= np.spacing(np.float32(abs(ref))), (r, e)


def test_nvfp4_router_logit_scale():
    # The generator's scale2 gives weights of variance about 1/h, so logits of
    # N(0,1) rows have a standard deviation near 1, as with the fp32 router.
    import synth
    shape = synth.CONFIGS["c2_e128_verify2"]
    t = synth.router_nvfp4(shape)
    L = RT.router_logits(synth.activations(shape, 0), t)
    assert 0.7 < float(np.std(L)) < 1.4


def test_topk_margin_constructed_keys():
    keys = np.array([3.0, 1.0, 2.0, 2.0], np.float32)
    assert RT.topk_margin(keys, 1) == 1.0  # 3 vs 2
    assert RT.topk_margin(keys, 2) == 0.0  # an exact tie between ranks 2 and 3
    assert RT.topk_margin(keys, 3) == 1.0  # 2 vs 1
    assert RT.topk_margin(keys, 4) == math.inf


def test_topk_margin_is_best_subset_gap():
    # Brute force over every k-subset S: the margin is the largest value of
    # min(keys in S) - max(keys outside S), reached by the selected set.
    import itertools
    rng = np.random.default_rng(21)
    for trial in range(60):
        E = int(rng.integers(2, 8))
        k = int(rng.integers(1, E))
        keys = rng.standard_normal(E).astype(np.float32)
        best = max(min(float(keys[e]) for e in S) - max(float(keys[e]) for e in range(E) if e not in S)
                   for S in itertools.combinations(range(E), k))
        assert RT.topk_margin(keys, k) == best
        sel = RT.select_topk(keys, k)
        assert min(float(keys[e]) for e in sel) - max(float(keys[e]) for e in range(E) if e not in sel) == best


def test_selection_keys_by_route_kind():
    L = np.array([[0.0, 1.0, -2.0]], np.float32)
    bias = np.array([0.25, -0.125, 0.0], np.float32)
    assert np.array_equal(RT.selection_keys(L, None, RT.ROUTE_SOFTMAX), L)
    # sigmoid(0) = 0.5 exactly: key 0.75; the others through sigmoid_keys
    k = RT.selection_keys(L, bias, RT.ROUTE_SIGMOID_BIAS)
    assert k[0, 0] == np.float32(0.75)
    assert np.array_equal(k, RT.sigmoid_keys(L, bias))
