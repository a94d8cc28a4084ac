"""Pins for the oracle's calibration statistics and scale rules."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.calibration import band_counts, ceil_bf16, scale_from_amax, AMAX_448, CEIL_BF16, SAFETY_1P3
from oracle.kvcache import calibrate_amax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "calibration_rules.json")


def all_bf16() -> np.ndarray:
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def bf16_pattern(v: float) -> int:
    return int(np.float32(v).view(np.uint32) >> 16)


@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_band_counts_closed_form_over_all_bf16(scale):
    """With a power-of-two scale y = x / s is exact, so the bands follow from
    the bf16 bit layout alone: clipped = finite magnitudes above 448 s plus
    infinity (patterns pattern(448 s)+1 .. 0x7F80 per sign); flushed = nonzero
    magnitudes up to 2^-10 s, where e4m3's smallest subnormal is 2^-9 and the
    tie at 2^-10 rounds to the even code 0 (patterns 1 .. pattern(2^-10 s))."""
    x = all_bf16()
    clipped, flushed = band_counts(x, scale)
    assert clipped == 2 * (0x7F80 - bf16_pattern(448 * scale))
    assert flushed == 2 * bf16_pattern(2.0 ** -10 * scale)
    assert (clipped, flushed) == ((30528, 29952) if scale == 1.0 else (30272, 30208))


def test_band_counts_rows_slots_nan_zero():
    x = np.array([[500.0, 1e-4, 0.0, -0.0], [np.nan, np.inf, -np.inf, 3.0], [-449.0, -1e-6, 447.0, 1.0]],
                 np.float32)
    assert band_counts(x, 1.0) == (4, 2)          # 500, inf, -inf, -449; 1e-4, -1e-6
    assert band_counts(x, 1.0, slot_mapping=[0, -1, 5]) == (2, 2)
    assert band_counts(x, 4.0) == (2, 2)          # only the infinities clip at scale 4
    assert band_counts(x[:0], 1.0) == (0, 0)


def test_ceil_bf16_rule_is_smallest_bf16_keeping_the_range():
    """For every positive finite bf16 amax the scale is bf16, at least amax/448
    in exact arithmetic, and the next bf16 below it is not."""
    x = all_bf16()
    pos = x[(x > 0) & np.isfinite(x)]
    for a in pos:
        s = scale_from_amax(a, CEIL_BF16)
        bits = int(np.float32(s).view(np.uint32))
        assert bits & 0xFFFF == 0
        need = Fraction(float(a)) / 448
        assert Fraction(float(s)) >= need
        below = np.array(bits - 0x10000, dtype=np.uint32).view(np.float32)[()]
        assert Fraction(float(below)) < need
    assert scale_from_amax(448.0, CEIL_BF16) == 1.0
    assert scale_from_amax(449.0, CEIL_BF16) == np.float32(1.0 + 2.0 ** -7)
    assert ceil_bf16(np.inf) == np.inf and ceil_bf16(0.0) == 0.0


def test_safety_rule_values_printed_by_the_page():
    g = json.load(open(GOLDEN))["safety_rule"]
    s = scale_from_amax(g["v_amax"], SAFETY_1P3)
    assert round(float(s), g["printed_decimals"]) == g["v_scale_printed"]
    for a in g["k_amax"]:
        assert scale_from_amax(a, SAFETY_1P3) == g["k_scale"]
    assert scale_from_amax(0.0, SAFETY_1P3) == 1.0
    assert scale_from_amax(448.0 / 1.3, SAFETY_1P3) == 1.0


def test_rules_around_the_amax_and_amax448_matches_calibration():
    """Stored at its own scale, the amax never clips under SAFETY_1P3 (1.3
    margin); under AMAX_448 and CEIL_BF16 it lands on 448 up to the fp32
    roundings of the quotient, the reciprocal and the product (so the clamp may
    catch it by an ulp, with the same e4m3 code 448). The AMAX_448 rule is the
    calibration's scale."""
    from oracle.kvcache import quantize_e4m3, reciprocal_f32
    rng = np.random.default_rng(4)
    ulp_clips = 0
    for a in np.concatenate([[1272.0, 812.0, 55.8, 1e-3, 3e4], rng.lognormal(2, 3, 400)]).astype(np.float32):
        pair = np.array([a, -a], np.float32)
        assert band_counts(pair, scale_from_amax(a, SAFETY_1P3))[0] == 0
        for rule in (AMAX_448, CEIL_BF16):
            s = scale_from_amax(a, rule)
            y = abs(float(np.float32(a * reciprocal_f32(s))))
            assert y <= 448.0 * (1 + 2.0 ** -21)
            assert list(quantize_e4m3(pair, s)) == [0x7E, 0xFE] or y < 448.0
            ulp_clips += band_counts(pair, s)[0]
        assert scale_from_amax(a, AMAX_448) == calibrate_amax(np.array([a], np.float32))[1]
    assert ulp_clips > 0          # the rounding case does occur
    t2 = json.load(open(GOLDEN))
    for a in t2["tier2_v_amax"]:
        assert band_counts(np.array([a, -a], np.float32), 3.0)[0] == t2["tier2_clip_at_scale_3"]
