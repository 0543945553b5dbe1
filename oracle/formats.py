"""Element formats of the layer's tensors, decoded to float64.

Pinned by tests/test_oracle_formats.py:
* E2M1 against the OCP MX v1.0 FP4 value table (tests/golden/e2m1_ocp_mx.txt),
* E4M3FN against torch's float8_e4m3fn -> float32 conversion (all 256 bytes),
* bf16 widening/rounding against torch's bfloat16 conversions,
* NVFP4 layout against hand-decoded bytes (tests/golden/nvfp4_layout.txt)
  and closed-form all-ones / one-hot matrices.

The pages only name the weight format NVFP4 (the token-major page serves its
NVFP4 experts untransposed, through pointer tables of packed codes, scales
and ``scale2`` values).  The readings used here: a projection [n, k] is stored
K-contiguous ("untransposed"), two E2M1 codes per byte with the even column in
the low nibble, one E4M3FN scale per 16 consecutive columns in a row-major
[n, k/16] array, and one fp32 per-tensor ``scale2``.
"""

from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """OCP MX FP4 (E2M1): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.

    Exponent field 0 is subnormal: value = m * 2^(1-1) * 0.5 = 0.5*m.
    Otherwise value = 2^(e-1) * (1 + m/2).  No Inf/NaN encodings.
    """
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e4m3fn_value(byte: int) -> float:
    """OCP 8-bit FP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal: (m/8) * 2^-6.  S.1111.111 is NaN; there is
    no infinity, so S.1111.000..110 are ordinary normals up to 448.
    """
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    e = (byte >> 3) & 15
    m = byte & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3FN_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64: the bits are the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round to nearest fp32 (numpy's cast is IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bits.

    bf16 keeps the top 16 bits of the fp32 pattern; rounding adds half an
    ulp of the kept part (0x7FFF) plus the kept lsb for the tie-to-even case.
    Inputs here are finite.
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def unpack_e2m1_codes(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """uint8 [n, k/2] -> codes uint8 [n, k]; column 2j is the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    return codes


def dequant_nvfp4(packed: np.ndarray, scales: np.ndarray, scale2: float, n: int, k: int) -> np.ndarray:
    """NVFP4 [n, k] -> float64: W[i, t] = e2m1(code[i, t]) * e4m3(scale[i, t//16]) * scale2."""
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    codes = unpack_e2m1_codes(packed, n, k)
    elem = np.take(E2M1_TABLE, codes)                                   # [n, k]
    s = np.take(E4M3FN_TABLE, np.asarray(scales, dtype=np.uint8).reshape(n, k // 16))
    w = elem.reshape(n, k // 16, 16) * s[:, :, None]                  # scale per 16 columns
    return w.reshape(n, k) * float(scale2)
