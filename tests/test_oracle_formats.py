"""Pins for the oracle's element formats and NVFP4 layout (CPU only)."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_e2m1_golden():
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            table[int(c)] = float(v)
    return table


def test_e2m1_matches_ocp_table():
    gold = _load_e2m1_golden()
    assert sorted(gold) == list(range(16))
    for c in range(16):
        v = F.E2M1_TABLE[c]
        assert v == gold[c], (c, v, gold[c])
        assert np.signbit(v) == np.signbit(gold[c]), c  # -0.0 for code 8


def test_e2m1_invariants():
    t = F.E2M1_TABLE
    assert np.all(np.diff(t[:8]) > 0)                # magnitudes increase with the code
    assert np.array_equal(t[8:], -t[:8])             # bit 3 is the sign
    assert t[7] == 6.0 and t[1] == 0.5               # max normal, the subnormal


def test_e4m3fn_all_bytes_match_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    ours = F.E4M3FN_TABLE
    nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
    assert np.array_equal(nan_ref, nan_ours)
    assert np.flatnonzero(nan_ours).tolist() == [0x7F, 0xFF]
    assert np.array_equal(ref[~nan_ref], ours[~nan_ours])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(ours[~nan_ours]))


def test_e2m1_times_e4m3_is_exact_in_bf16():
    # Every product of an E2M1 value and a finite E4M3FN scale has <= 6
    # significant bits and lies in [2^-10, 2688]: exact in bf16 (8 bits).
    fin = F.E4M3FN_TABLE[np.isfinite(F.E4M3FN_TABLE)]
    prod = (F.E2M1_TABLE[:, None] * fin[None, :]).reshape(-1)
    as_bf16 = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, prod)


def test_bf16_widen_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 65536, size=20000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_to_f64(bits), ref)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(50000).astype(np.float32) * np.float32(100)
    # exact ties: fp32 values halfway between two bf16 values
    ties = ((rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, 3.0e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(x), ref)


def _load_layout_golden():
    packed = np.zeros((2, 16), np.uint8)
    scales = np.zeros((2, 2), np.uint8)
    expect = np.zeros((2, 32), np.float64)
    with open(os.path.join(GOLDEN, "nvfp4_layout.txt")) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0] == "packed":
                packed[int(p[1])] = [int(v, 16) for v in p[2:]]
            elif p[0] == "scales":
                scales[int(p[1])] = [int(v, 16) for v in p[2:]]
            elif p[0] == "expect":
                expect[int(p[1]), int(p[2])] = float(p[3])
            elif p[0] == "expect_row":
                expect[int(p[1]), int(p[3]):int(p[4]) + 1] = float(p[5])
    return packed, scales, expect


def test_nvfp4_layout_golden():
    packed, scales, expect = _load_layout_golden()
    w = F.dequant_nvfp4(packed, scales, 1.0, 2, 32)
    assert np.array_equal(w, expect)
    assert np.signbit(w[0, 6])  # code 8 is -0.0


def test_nvfp4_all_ones_and_scale2():
    n, k = 3, 64
    packed = np.full((n, k // 2), 0x22, np.uint8)   # both nibbles code 2 = 1.0
    scales = np.full((n, k // 16), 0x38, np.uint8)  # 1.0
    assert np.array_equal(F.dequant_nvfp4(packed, scales, 1.0, n, k), np.ones((n, k)))
    assert np.array_equal(F.dequant_nvfp4(packed, scales, 0.25, n, k), np.full((n, k), 0.25))


def test_nvfp4_one_hot_columns():
    # Row i holds 1.0 at column perm[i] only: checks row/column placement.
    n, k = 16, 64
    perm = np.random.default_rng(3).permutation(k)[:n]
    codes = np.zeros((n, k), np.uint8)
    codes[np.arange(n), perm] = 2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((n, k // 16), 0x38, np.uint8)
    w = F.dequant_nvfp4(packed, scales, 1.0, n, k)
    ref = np.zeros((n, k))
    ref[np.arange(n), perm] = 1.0
    assert np.array_equal(w, ref)
