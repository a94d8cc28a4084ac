"""Calibration statistics and scale-rule variants, in plain numpy.

Test infrastructure only (see the package header).

Band counters (vLLM PR 54705 evidence, "Tier 2: KV value range at unity
scale": exact e4m3 band counters of the values actually stored, at scales 1.0
and 3.0, as clip and flush-to-zero rates; the same section records that an
earlier "subnormal" counter had measured values below e4m3's smallest
magnitude). At a scale s, with y = fp32(x) * fp32(1/s) as the store computes
it:
  clipped = stored values with |y| > 448, the ones the clamp changes
            (infinities included, NaN excluded);
  flushed = nonzero stored values whose e4m3 code is +0 or -0 (NaN excluded).
Rows whose slot is negative are not stored and not counted.

Scale rules, applied to a running amax:
  AMAX_448   = fp32(amax) / fp32(448) in fp32 (Qwen3.8-27B-FP8-KVcal model
               card, scale table);
  CEIL_BF16  = the smallest bf16 value >= fp32(amax) / fp32(448), stored as
               fp32 (same card, "Rebuild / reproduce": ceil_to_bfloat16, the
               smallest bf16-representable scale that keeps the range);
  SAFETY_1P3 = max(1, amax * 1.3 / 448) evaluated in fp64 left to right and
               rounded to fp32 (vLLM PR 54705 evidence, "Tier 4", paragraph on
               the calibration utility: the rule rewidened to a 1.3 safety
               factor with a floor of 1).
Readings where the pages are silent: the precisions just stated (the card's
script and the PR's utility are not printed).

Pins: tests/test_oracle_calibration.py (band counts over all 65,536 bf16
patterns at scales 1 and 2 from the bf16 bit layout; CEIL_BF16 against its
definition in exact rationals for every positive finite bf16 amax; the worked
values the PR page prints for SAFETY_1P3, tests/golden/calibration_rules.json).
"""
from __future__ import annotations

import numpy as np

from .codecs import E4M3_MAX
from .kvcache import quantize_e4m3, reciprocal_f32

AMAX_448, CEIL_BF16, SAFETY_1P3 = 0, 1, 2


def _stored_rows(x: np.ndarray, slot_mapping) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    rows = x.reshape(x.shape[0], int(np.prod(x.shape[1:], dtype=np.int64))) if x.ndim > 1 else x.reshape(-1, 1)
    if slot_mapping is not None:
        rows = rows[np.asarray(slot_mapping, dtype=np.int64) >= 0]
    return rows


def band_counts(x: np.ndarray, scale: float, slot_mapping=None):
    """(clipped, flushed) counts of the stored rows of x [rows, ...] at scale."""
    rows = _stored_rows(x, slot_mapping)
    nan = np.isnan(rows)
    with np.errstate(over="ignore", invalid="ignore"):
        y = rows * reciprocal_f32(scale)
    clipped = int(np.count_nonzero(~nan & (np.abs(y) > np.float32(E4M3_MAX))))
    codes = quantize_e4m3(rows, scale)
    flushed = int(np.count_nonzero(~nan & (rows != 0) & ((codes & 0x7F) == 0)))
    return clipped, flushed


def ceil_bf16(v) -> np.float32:
    """The smallest bf16 value >= v, for v >= 0 (inf stays inf)."""
    b = int(np.asarray(v, dtype=np.float32).view(np.uint32))
    if b & 0xFFFF:
        b = (b & 0xFFFF0000) + 0x10000
    return np.array(b, dtype=np.uint32).view(np.float32)[()]


def scale_from_amax(amax, rule: int) -> np.float32:
    """The scale of a running amax under one of the three rules."""
    a = np.float32(amax)
    if rule == AMAX_448:
        return np.float32(a / np.float32(E4M3_MAX))
    if rule == CEIL_BF16:
        return ceil_bf16(a / np.float32(E4M3_MAX))
    if rule == SAFETY_1P3:
        return np.float32(max(1.0, float(a) * 1.3 / 448.0))
    raise ValueError("unknown rule %r" % (rule,))
