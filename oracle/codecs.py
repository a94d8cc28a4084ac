"""Number formats: OCP e4m3 (E4M3FN), e2m1 (FP4) and bf16 rounding.

Test infrastructure only (see the package header).

* e4m3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the only
  NaN pattern is S.1111.111; largest finite value 448 (vLLM PR 54705,
  "Purpose": the store clamp targets the e4m3 finite range; "Tier 0": log2 of
  the e4m3 maximum 448). Rounding is IEEE round-to-nearest-even (the pages do
  not name a mode; this is the plain IEEE reading). Conversion itself does not
  saturate: a magnitude above 464 becomes NaN, as an IEEE conversion to a
  format without infinity does. Saturation is the store's explicit clamp.
* e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} (local-inference-lab/vllm PR 189, "Why": record
  values are E2M1). Round-to-nearest-even on the code, sign kept.
* bf16: the upper half of an fp32, round-to-nearest-even.

Pins: brute-force nearest-value search over every code, torch's independent
float8_e4m3fn cast, and worked grid values (tests/test_oracle_codecs.py).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
E4M3_MIN_NORMAL_EXP = -6   # smallest normal 2^-6
E4M3_MANT_BITS = 3
E4M3_BIAS = 7


def _e4m3_value(code: int) -> float:
    """Value of one e4m3 code from its bit fields."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** (1 - E4M3_BIAS - E4M3_MANT_BITS)  # m * 2^-9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to e4m3 codes (RNE, no saturation).

    |y| below 2^-6 is a subnormal: code = rint(|y| * 2^9) (8 is the smallest
    normal, whose code is also 8). Otherwise e = floor(log2|y|) and the
    4-bit significand m = rint(|y| / 2^(e-3)) in [8, 16]; m = 16 carries into
    the next binade. Magnitudes rounding past 448 give the NaN code.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    sign = np.signbit(y).astype(np.uint8) << 7
    nan = np.isnan(y)
    a_safe = np.where(nan | np.isinf(a), 0.0, a)
    sub = a_safe < 2.0 ** E4M3_MIN_NORMAL_EXP
    code_sub = np.rint(a_safe * 2.0 ** 9)
    _, ex = np.frexp(np.where(sub, 1.0, a_safe))   # a = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1                    # floor(log2 a)
    m = np.rint(np.where(sub, 8.0, a_safe) / np.exp2((e - 3).astype(np.float64)))
    carry = m >= 16.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8.0, m)
    code_norm = ((e + E4M3_BIAS) << 3) | (m.astype(np.int64) - 8)
    code = np.where(sub, code_sub.astype(np.int64), code_norm)
    overflow = np.isinf(a) | (code > 0x7E)
    code = np.where(overflow | nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_TABLE = np.concatenate([E2M1_GRID, -E2M1_GRID])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15) -> float64 values."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """Round values already clipped to [-6, 6] to e2m1 codes (RNE on the code).

    Within each binade the grid is evenly spaced, so rounding is numpy's rint
    (half to even) on the scaled magnitude: step 0.5 below 2, step 1 in [2, 4),
    step 2 in [4, 6]. The even integer there is the even code.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    sign = np.signbit(y).astype(np.uint8) << 3
    c0 = np.rint(a * 2.0)                # codes 0..4 cover 0, 0.5, 1, 1.5, 2
    c1 = np.rint(a) + 2.0                # 2 -> 4, 3 -> 5, 4 -> 6
    c2 = np.rint(a * 0.5) + 4.0          # 4 -> 6, 6 -> 7
    code = np.where(a < 2.0, c0, np.where(a < 4.0, c1, c2))
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.
    NaN stays NaN."""
    x = np.array(x, dtype=np.float32)
    shape = x.shape
    flat = x.reshape(-1)
    bits = flat.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(flat), flat, out).reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)
