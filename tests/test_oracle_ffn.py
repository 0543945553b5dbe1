"""Pins for the oracle's expert FFN (CPU only)."""

import math

import numpy as np

from oracle import ffn as FF
from oracle.formats import E2M1_TABLE, E4M3FN_TABLE, bf16_to_f64
from synth import Nvfp4Tensor


def pack(codes, scale_bytes, scale2=1.0):
    codes = np.asarray(codes, np.uint8)
    n, k = codes.shape
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return Nvfp4Tensor(n, k, packed, np.asarray(scale_bytes, np.uint8).reshape(n, k // 16), scale2)


def bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def one_hot(n, k, cols, code=2):
    c = np.zeros((n, k), np.uint8)
    c[np.arange(n), cols] = code
    return c


def test_all_ones_closed_form():
    h, I = 64, 32
    x = bf16_bits(np.random.default_rng(1).standard_normal(h) * 0.1)
    ones = lambda n, k: pack(np.full((n, k), 2), np.full((n, k // 16), 0x38))
    y = FF.ffn_nvfp4(ones(I, h), ones(I, h), ones(h, I), bf16_to_f64(x)[None])[0]
    s = float(np.float32(bf16_to_f64(x).sum()))
    a = float(np.float32(s / (1.0 + math.exp(-s)) * s))
    assert np.all(y == np.float32(I * a))


def test_one_hot_closed_form():
    # gate row i picks x[sg[i]], up row i picks x[su[i]], down row n picks a[sd[n]]:
    # y[n] = silu(x[sg[sd[n]]]) * x[su[sd[n]]].  Different permutations catch a
    # swapped gate/up, a transposed projection or a wrong row index.
    h, I = 48, 32
    rng = np.random.default_rng(2)
    sg, su = rng.permutation(h)[:I], rng.permutation(h)[:I]
    sd = rng.integers(0, I, size=h)
    x = bf16_bits(rng.standard_normal(h))
    xf = bf16_to_f64(x)
    one = lambda n, k, cols: pack(one_hot(n, k, cols), np.full((n, k // 16), 0x38))
    y = FF.ffn_nvfp4(one(I, h, sg), one(I, h, su), one(h, I, sd), xf[None])[0]
    g, v = xf[sg[sd]], xf[su[sd]]
    ref = np.array([np.float32(gi / (1 + math.exp(-gi)) * vi) for gi, vi in zip(g, v)], np.float32)
    assert np.array_equal(y, ref)


def test_scaled_one_hot_uses_block_scale():
    # code 3 (1.5) with block scale 0x40 (2.0) and scale2 0.5 -> weight 1.5
    h, I = 32, 16
    cols = np.arange(I) * 2
    gate = pack(one_hot(I, h, cols, code=3), np.full((I, h // 16), 0x40), 0.5)
    up = pack(one_hot(I, h, cols, code=2), np.full((I, h // 16), 0x38))
    down = pack(one_hot(h, I, np.arange(h) % I, code=2), np.full((h, I // 16), 0x38))
    x = bf16_bits(np.linspace(-2, 2, h))
    xf = bf16_to_f64(x)
    y = FF.ffn_nvfp4(gate, up, down, xf[None])[0]
    g = 1.5 * xf[cols]
    a = np.array([np.float32(gi / (1 + math.exp(-gi)) * vi) for gi, vi in zip(g, xf[cols])])
    assert np.array_equal(y, a[np.arange(h) % I].astype(np.float32))


def test_random_expert_matches_exact_sums():
    h, I = 64, 48
    rng = np.random.default_rng(3)
    mk = lambda n, k: pack(rng.integers(0, 16, (n, k)), rng.integers(0x20, 0x48, (n, k // 16)))
    gate, up, down = mk(I, h), mk(I, h), mk(h, I)
    xf = bf16_to_f64(bf16_bits(rng.standard_normal(h)))
    y = FF.ffn_nvfp4(gate, up, down, xf[None])[0]

    def elem(t, i, j):  # decode one weight straight from the bytes
        byte = t.packed[i, j // 2]
        code = (byte >> 4) if (j & 1) else (byte & 15)
        return E2M1_TABLE[code] * E4M3FN_TABLE[t.scales[i, j // 16]] * t.scale2

    g = [np.float32(math.fsum(elem(gate, i, t) * xf[t] for t in range(h))) for i in range(I)]
    v = [np.float32(math.fsum(elem(up, i, t) * xf[t] for t in range(h))) for i in range(I)]
    a = [np.float32(float(gi) / (1 + math.exp(-float(gi))) * float(vi)) for gi, vi in zip(g, v)]
    ref = np.array([np.float32(math.fsum(elem(down, n, i) * float(a[i]) for i in range(I)))
                    for n in range(h)], np.float32)
    # float64 BLAS sums vs exact sums: equal after fp32 rounding up to one ulp at a boundary
    diff = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    assert np.all(diff <= np.spacing(np.abs(ref)).astype(np.float64))
    assert np.count_nonzero(diff) <= 1
