"""NVFP4 368-byte MLA latent record and decode attention over it.

Test infrastructure only (see the package header).

Source: local-inference-lab/vllm PR 189, "mla: wire dynamic per-token NVFP4
scaling and cache ABI" (commit message and "Why"): the compressed latent is
stored as e2m1 values with E4M3 scales per group, next to an fp8 RoPE part; a
per-token fp32 second-level (outer) scale derived from the token's amax is
written into existing padding at record bytes [292, 296), the record stays
368 bytes, and readers take the outer scale from the record instead of a
per-layer launch scalar.

Readings where the page is silent (all fp32 arithmetic, correctly rounded):
  * group = 16 latent elements (32 groups for the 512-dim latent);
  * s2 = amax / 2688 with 2688 = 6 * 448, so the largest group scale lands on
    the e4m3 maximum; amax = 0 gives s2 = 0 and all-zero codes;
  * group scale code sg = e4m3_RNE(min(ag / fp32(6 * s2), 448)), ag = the
    group's amax; dg = fp32(dec(sg) * s2);
  * value codes: dg = 0 gives +0 codes for the whole group, otherwise
    e2m1_RNE(clip(fp32(x * fp32(1/dg)), -6, 6)), sign kept;
  * the 64 RoPE dims use the e4m3 store quantizer with a per-tensor rope scale;
  * byte layout: [0,256) values, element 2i in the low nibble of byte i and
    element 2i+1 in the high nibble; [256,288) group-scale codes; [288,292)
    zero; [292,296) s2 as little-endian fp32; [296,304) zero; [304,368) RoPE
    codes. Only the 368-byte size and the [292,296) position come from the
    page: the rest of the layout is parity unpinned (self-consistent only).
Decode: latent = e2m1(v) * e4m3(sg) * s2 and RoPE = e4m3(r) * rope_scale;
attention runs with one KV head, K = [latent ; RoPE] (576 dims), V = latent
(512 dims), on bf16 Q that is not quantized.

Static outer scale (same page, "Why": with an implicit outer scale of 1.0,
low-magnitude layers put many group scales in E4M3's subnormal range; the
commit message: the earlier writer's outer scale was statically 1.0, or a
per-layer calibrated constant): encode_records(..., static_s2=c) writes the
same record with s2 = c for every token, for the A/B against the per-token
scale. Prefill (same page, "Changes" and "Validation": the readers apply the
per-token scale in decode and in the multitile prefill): query i of a
sequence with Lq new tokens and L keys sits at position L - Lq + i and attends
keys j <= its position, with decode's arithmetic. mla_exact is attention
over the unquantized tokens, the reference both records are judged against.

Pins: tests/test_oracle_nvfp4.py (e2m1 brute force and tie set, a token with
amax 168 whose scales are exact, power-of-two invariance, s2 read-back,
no subnormal group scales on the layer-std range; static s2 equal to a
token's own s2 gives its dynamic record, static 1.0 puts low-magnitude group
scales into subnormals; every prefill row equals decode over the sequence cut
at its position; on tokens the record holds exactly, decode over the records
equals mla_exact).
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode
from .kvcache import quantize_e4m3

RECORD_BYTES = 368
LATENT = 512
ROPE = 64
GROUP = 16
NGROUPS = LATENT // GROUP
OFF_VALUES = 0
OFF_GSCALE = 256
OFF_S2 = 292
OFF_ROPE = 304
S2_DIVISOR = 2688.0   # 6 (e2m1 max) * 448 (e4m3 max)


def encode_records(x: np.ndarray, rope_scale: float = 1.0, static_s2=None) -> np.ndarray:
    """bf16 tokens (as float32) [T, 576] -> uint8 records [T, 368]. static_s2:
    one outer scale for every token instead of the per-token amax / 2688."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    lat = x[:, :LATENT]
    rope = x[:, LATENT:LATENT + ROPE]
    rec = np.zeros((T, RECORD_BYTES), dtype=np.uint8)
    amax = np.max(np.abs(lat), axis=1) if T else np.zeros(0, np.float32)
    if static_s2 is None:
        s2 = (amax / np.float32(S2_DIVISOR)).astype(np.float32)
    else:
        s2 = np.full(T, np.float32(static_s2), dtype=np.float32)
    d = (np.float32(6.0) * s2).astype(np.float32)
    g = lat.reshape(T, NGROUPS, GROUP)
    ag = np.max(np.abs(g), axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (ag / d[:, None]).astype(np.float32)
    ratio = np.where((amax[:, None] > 0) & (s2[:, None] > 0), ratio, np.float32(0.0))
    ratio = np.minimum(ratio, np.float32(448.0))
    sg = e4m3_encode(ratio)
    dg = (e4m3_decode(sg).astype(np.float32) * s2[:, None]).astype(np.float32)
    nz = dg != 0
    with np.errstate(divide="ignore"):
        r = np.where(nz, np.float32(1.0) / np.where(nz, dg, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    y = (g * r[:, :, None]).astype(np.float32)
    y = np.clip(y, np.float32(-6.0), np.float32(6.0))
    codes = np.where(nz[:, :, None], e2m1_encode(y), np.uint8(0)).reshape(T, LATENT)
    rec[:, OFF_VALUES:OFF_VALUES + LATENT // 2] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    rec[:, OFF_GSCALE:OFF_GSCALE + NGROUPS] = sg
    rec[:, OFF_S2:OFF_S2 + 4] = s2.astype("<f4").view(np.uint8).reshape(T, 4)
    rec[:, OFF_ROPE:OFF_ROPE + ROPE] = quantize_e4m3(rope, rope_scale)
    return rec


def record_s2(rec: np.ndarray) -> np.ndarray:
    """Per-token outer scale read back from bytes [292, 296)."""
    rec = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8)[..., OFF_S2:OFF_S2 + 4])
    return rec.view("<f4")[..., 0]


def decode_records(rec: np.ndarray, rope_scale: float = 1.0):
    """uint8 records [N, 368] -> (latent fp64 [N, 512], rope fp64 [N, 64])."""
    rec = np.asarray(rec, dtype=np.uint8)
    N = rec.shape[0]
    packed = rec[:, OFF_VALUES:OFF_VALUES + LATENT // 2]
    codes = np.empty((N, LATENT), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = e2m1_decode(codes).reshape(N, NGROUPS, GROUP)
    gsc = e4m3_decode(rec[:, OFF_GSCALE:OFF_GSCALE + NGROUPS])
    s2 = record_s2(rec).astype(np.float64)
    latent = (vals * gsc[:, :, None]).reshape(N, LATENT) * s2[:, None]
    rope = e4m3_decode(rec[:, OFF_ROPE:OFF_ROPE + ROPE]) * float(rope_scale)
    return latent, rope


def new_pool(num_pages: int, page_size: int = 16, fill: int = 0x7F) -> np.ndarray:
    return np.full((num_pages, page_size, RECORD_BYTES), fill, dtype=np.uint8)


def store_records(pool: np.ndarray, x: np.ndarray, slot_mapping: np.ndarray,
                  rope_scale: float = 1.0, static_s2=None) -> None:
    """Encode tokens [T, 576] and write each record at its slot (in place)."""
    page_size = pool.shape[1]
    slot = np.asarray(slot_mapping, dtype=np.int64)
    keep = slot >= 0
    rec = encode_records(np.asarray(x, dtype=np.float32)[keep], rope_scale, static_s2)
    s = slot[keep]
    pool[s // page_size, s % page_size, :] = rec


def mla_decode(q: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
               seq_lens: np.ndarray, softmax_scale: float, rope_scale: float = 1.0,
               seqs=None) -> np.ndarray:
    """One query per sequence over its NVFP4 records. q: [B, Hq, 576] float32
    (bf16 values, not quantized). Returns fp64 [B, Hq, 512]."""
    B, Hq, _ = q.shape
    page_size = pool.shape[1]
    out = np.zeros((B, Hq, LATENT), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        if L == 0:
            continue
        pos = np.arange(L, dtype=np.int64)
        page = np.asarray(block_table[b], dtype=np.int64)[pos // page_size]
        rec = pool[page, pos % page_size, :]
        latent, rope = decode_records(rec, rope_scale)
        kfull = np.concatenate([latent, rope], axis=1)
        qb = np.asarray(q[b], dtype=np.float64)
        s = (qb @ kfull.T) * float(softmax_scale)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[b] = (w @ latent) / w.sum(axis=1, keepdims=True)
    return out


def mla_prefill(q: np.ndarray, cu_q_lens: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                seq_lens: np.ndarray, softmax_scale: float, rope_scale: float = 1.0,
                rows=None) -> np.ndarray:
    """New queries of sequence b: rows cu_q_lens[b] .. cu_q_lens[b+1]-1 of
    q [sumQ, Hq, 576] (float32 bf16 values), query i at position L - Lq + i,
    causal over the sequence's records. ``rows`` restricts the computed rows
    (global indices); others stay zero. Returns fp64 [sumQ, Hq, 512]."""
    nrows, Hq, _ = q.shape
    page_size = pool.shape[1]
    out = np.zeros((nrows, Hq, LATENT), dtype=np.float64)
    want = None
    if rows is not None:
        want = np.zeros(nrows, dtype=bool)
        want[np.asarray(rows, dtype=np.int64)] = True
    for b in range(len(seq_lens)):
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        L = int(seq_lens[b])
        idx = np.arange(r0, r1)
        if want is not None:
            idx = idx[want[r0:r1]]
        if idx.size == 0 or L == 0:
            continue
        pos_all = np.arange(L, dtype=np.int64)
        page = np.asarray(block_table[b], dtype=np.int64)[pos_all // page_size]
        latent, rope = decode_records(pool[page, pos_all % page_size, :], rope_scale)
        kfull = np.concatenate([latent, rope], axis=1)
        qpos = L - (r1 - r0) + (idx - r0)
        for r, p in zip(idx, qpos):
            s = (np.asarray(q[r], dtype=np.float64) @ kfull[:p + 1].T) * float(softmax_scale)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[r] = (w @ latent[:p + 1]) / w.sum(axis=1, keepdims=True)
    return out


def mla_exact(q: np.ndarray, kv: np.ndarray, seq_lens: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Attention over the unquantized tokens (the reference of the static /
    per-token outer-scale A/B of local-inference-lab/vllm PR 189, "Why"): kv
    [T, 576] float32 tokens of all sequences back to back, K = the 576 dims,
    V = the 512 latent dims, one query per sequence. Returns fp64 [B, Hq, 512]."""
    B, Hq, _ = q.shape
    out = np.zeros((B, Hq, LATENT), dtype=np.float64)
    start = 0
    for b in range(B):
        L = int(seq_lens[b])
        k = np.asarray(kv[start:start + L], dtype=np.float64)
        start += L
        if L == 0:
            continue
        s = (np.asarray(q[b], dtype=np.float64) @ k.T) * float(softmax_scale)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[b] = (w @ k[:, :LATENT]) / w.sum(axis=1, keepdims=True)
    return out
