"""Pins for the oracle's number formats, independent of the oracle's own
encoder: brute-force nearest-value search over all codes, torch's float8 cast,
and values the pages state (e4m3 max 448, the 0.807 bound)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.codecs import (E4M3_TABLE, e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode,
                           bf16_round, bf16_bits_to_f32)
from oracle.kvcache import quantize_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def nearest_code_bruteforce(y: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3 value by exhaustive search, ties to the even code.
    Input must be finite and |y| <= 448."""
    y = np.asarray(y, dtype=np.float64)
    mags = E4M3_TABLE[:0x7F]                       # codes 0..126, all finite, >= 0
    a = np.abs(y)[:, None]
    dist = np.abs(a - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    codes = np.arange(0x7F)[None, :]
    # among tied candidates prefer the even code
    even = cand & (codes % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return (pick.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def test_page_constants_fixture():
    g = golden()
    assert g["e4m3_max"]["value"] == 448.0
    assert np.nanmax(E4M3_TABLE) == 448.0
    # log2(448) - 8: the largest lazy-rescale slack that never clips P
    assert abs(math.log2(g["e4m3_max"]["value"]) - g["p_prescale_exponent"]["value"]
               - g["rescale_threshold_bound"]["value"]) < 5e-4


def test_e4m3_table_structure():
    finite = E4M3_TABLE[~np.isnan(E4M3_TABLE)]
    assert finite.size == 254
    assert np.isnan(E4M3_TABLE[0x7F]) and np.isnan(E4M3_TABLE[0xFF])
    assert E4M3_TABLE[0x7E] == 448.0 and E4M3_TABLE[0xFE] == -448.0
    assert E4M3_TABLE[0x01] == 2.0 ** -9 and E4M3_TABLE[0x08] == 2.0 ** -6
    # positive codes are monotone in value
    pos = E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)


def all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    x = bf16_bits_to_f32(bits)
    return x[np.isfinite(x)]


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 20.0 / 448.0, 1272.0 / 448.0])
def test_quantizer_matches_bruteforce_all_bf16(scale):
    x = all_bf16_finite()
    got = quantize_e4m3(x, scale)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore"):
        y = np.clip(x * inv, np.float32(-448), np.float32(448))
    want = nearest_code_bruteforce(y)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("scale", [1.0, 3.0, 20.0 / 448.0])
def test_quantizer_matches_torch_cast(scale):
    x = all_bf16_finite()
    got = quantize_e4m3(x, scale)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore"):
        y = np.clip(x * inv, np.float32(-448), np.float32(448))
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_saturation_set():
    xs = np.array([448, 449, 463.9, 464, 465, 1000, 1272, 1e30, np.inf], dtype=np.float32)
    assert np.all(quantize_e4m3(xs, 1.0) == 0x7E)
    assert np.all(quantize_e4m3(-xs, 1.0) == 0xFE)


def test_encoder_nonsaturating_and_nan():
    # the bare conversion (no clamp) turns overflow into NaN, like torch's cast
    assert e4m3_encode(np.array([464.0]))[0] == 0x7E
    assert e4m3_encode(np.array([465.0]))[0] == 0x7F
    assert e4m3_encode(np.array([-np.inf]))[0] == 0xFF
    q = quantize_e4m3(np.array([np.nan], dtype=np.float32), 1.0)[0]
    assert q & 0x7F == 0x7F


def test_signed_zero_and_tiny():
    assert quantize_e4m3(np.array([-1e-5], dtype=np.float32), 1.0)[0] == 0x80
    assert quantize_e4m3(np.array([2.0 ** -10], dtype=np.float32), 1.0)[0] == 0x00  # tie -> even 0
    assert quantize_e4m3(np.array([3 * 2.0 ** -10], dtype=np.float32), 1.0)[0] == 0x02  # 1.5 ulp -> 2
    assert quantize_e4m3(np.array([5 * 2.0 ** -10], dtype=np.float32), 1.0)[0] == 0x02  # 2.5 ulp -> 2


def test_grid_round_trip_power_of_two_scales():
    codes = np.array([c for c in range(256) if not np.isnan(E4M3_TABLE[c])], dtype=np.uint8)
    vals = e4m3_decode(codes)
    for k in range(-8, 9):
        s = 2.0 ** k
        x = (vals * s).astype(np.float32)
        got = quantize_e4m3(x, s)
        assert np.array_equal(got, codes), k


def test_power_of_two_invariance():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 30).astype(np.float32)
    x = bf16_round(x)
    base = quantize_e4m3(x, 0.75)
    for k in (-6, -1, 1, 5):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        assert np.array_equal(quantize_e4m3(xs, 0.75 * 2.0 ** k), base)


def test_gaussian_round_trip_error_matches_pages_range():
    # The evidence document's Tier 2 table puts the e4m3 round-trip error of
    # real K/V at 2.3-2.6%; Gaussian data at unit scale lands in that band.
    g = golden()["round_trip_rel_err"]
    rng = np.random.default_rng(11)
    x = bf16_round(rng.standard_normal(200000).astype(np.float32))
    xh = e4m3_decode(quantize_e4m3(x, 1.0))
    rel = np.linalg.norm(xh - x) / np.linalg.norm(x)
    assert g["lo"] - 0.005 < rel < g["hi"] + 0.005


def test_e2m1_bruteforce():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    ys = np.linspace(-6, 6, 48001)
    ys = np.concatenate([ys, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, -0.0]])
    got = e2m1_encode(ys)
    a = np.abs(ys)[:, None]
    dist = np.abs(a - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    want = pick.astype(np.uint8) | (np.signbit(ys).astype(np.uint8) << 3)
    assert np.array_equal(got, want)


def test_e2m1_ties():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want_vals = np.array([0, 1, 1, 2, 2, 4, 4], dtype=np.float64)
    assert np.array_equal(e2m1_decode(e2m1_encode(ties)), want_vals)
    assert np.array_equal(e2m1_decode(e2m1_encode(-ties)), -want_vals)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1000,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 65504.5], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_round(x), want)
