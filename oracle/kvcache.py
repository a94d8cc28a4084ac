"""Quant-on-store into the paged e4m3 cache, and amax calibration.

Test infrastructure only (see the package header).

Store (vLLM PR 54705, "Purpose" quant-on-store bullet; evidence "Tier 1"
write-path paragraph): each element is multiplied by the reciprocal of the
per-tensor scale, clamped to [-448, 448] because a plain float-to-fp8 cast does
not saturate, and converted to e4m3. Reading taken where the page is silent:
the reciprocal is one fp32 division 1/scale done once, the product is an fp32
multiply, conversion is round-to-nearest-even, NaN stays NaN.

Cache layout (the pages only say the pool is raw uint8 viewed as e4m3, PR 54705
"Purpose" cache-plumbing bullet; the layout is this library's choice):
  K: u8 [num_pages][num_kv_heads][page_size][head_dim]
  V: u8 [num_pages][num_kv_heads][head_dim][page_size]   (token-minor)
  slot = page * page_size + offset; rows with slot < 0 are not stored.

Calibration (Qwen3.8-27B-FP8-KVcal model card, scale table: scale = amax/448
for k, v and q; "Rebuild / reproduce": the amax is a running maximum over
calls; vLLM PR 54705 "Tier 2": statistics cover exactly the stored rows):
amax is the largest |x| over rows whose slot is >= 0 (all rows when no slot
mapping is given), combined with the previous running value by max;
scale = fp32(amax) / fp32(448) in fp32.

Pins: tests/test_oracle_kvcache.py (saturation set, grid round trip,
power-of-two invariance, torch's independent e4m3 cast, amax closed forms).
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_encode, e4m3_decode, E4M3_MAX


def reciprocal_f32(scale: float) -> np.float32:
    """fp32(1 / scale) with one correctly rounded fp32 division."""
    return np.float32(1.0) / np.float32(scale)


def quantize_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """float32 values (bf16 inputs widened exactly) -> e4m3 codes."""
    inv = reciprocal_f32(scale)
    with np.errstate(over="ignore"):
        y = np.asarray(x, dtype=np.float32) * inv       # fp32 multiply, RNE
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y)


def new_cache(num_pages: int, num_kv_heads: int, page_size: int, head_dim: int,
              fill: int = 0x7F):
    """Fresh K and V pools, every byte set to ``fill``."""
    k = np.full((num_pages, num_kv_heads, page_size, head_dim), fill, dtype=np.uint8)
    v = np.full((num_pages, num_kv_heads, head_dim, page_size), fill, dtype=np.uint8)
    return k, v


def store_e4m3(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
               slot_mapping: np.ndarray, k_scale: float, v_scale: float) -> None:
    """Quantize K/V rows [T, Hkv, D] and write them at their slots (in place)."""
    page_size = k_cache.shape[2]
    slot = np.asarray(slot_mapping, dtype=np.int64)
    keep = slot >= 0
    slot = slot[keep]
    kq = quantize_e4m3(np.asarray(k, dtype=np.float32)[keep], k_scale)
    vq = quantize_e4m3(np.asarray(v, dtype=np.float32)[keep], v_scale)
    page, off = slot // page_size, slot % page_size
    k_cache[page, :, off, :] = kq
    # V is token-minor inside a page: [page][head][dim][offset]
    v_cache[page, :, :, off] = vq


def gather_tokens(k_cache: np.ndarray, v_cache: np.ndarray, block_table_row: np.ndarray,
                  length: int):
    """Codes of tokens 0..length-1 of one sequence: K, V as [L, Hkv, D]."""
    page_size = k_cache.shape[2]
    pos = np.arange(length, dtype=np.int64)
    page = np.asarray(block_table_row, dtype=np.int64)[pos // page_size]
    off = pos % page_size
    k = k_cache[page, :, off, :]
    v = v_cache[page, :, :, off]
    return k, v


def calibrate_amax(x: np.ndarray, slot_mapping=None, prev_amax: float = 0.0):
    """Running amax over stored rows of ``x`` [rows, ...] and the derived scale.

    Returns (amax as np.float32, scale as np.float32)."""
    x = np.asarray(x, dtype=np.float32)
    rows = x.reshape(x.shape[0], int(np.prod(x.shape[1:], dtype=np.int64)))
    if slot_mapping is not None:
        rows = rows[np.asarray(slot_mapping, dtype=np.int64) >= 0]
    amax = np.float32(prev_amax)
    if rows.size:
        amax = np.maximum(amax, np.max(np.abs(rows)))
    scale = np.float32(amax) / np.float32(E4M3_MAX)
    return np.float32(amax), np.float32(scale)
