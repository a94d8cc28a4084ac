"""Seeded generators: random draws, bf16 rounding and page layout only.

Every array is produced from ``numpy.random.Generator(PCG64(seed))`` in a fixed
draw order (Q, K, V, outlier mask/magnitudes/signs, page permutation), so the
oracle and the GPU path see the same bytes for the same seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16
POISON_BYTE = 0x7F  # e4m3 NaN: a read of an unused page poisons the result


def bf16(x: np.ndarray) -> torch.Tensor:
    """Round float32 data to bf16 (round-to-nearest-even, torch's CPU cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _rms_normed(rng: np.random.Generator, shape, amax_target: float) -> np.ndarray:
    """N(0,1) rows normalised to unit RMS over the last axis, then one global
    factor so the tensor's largest magnitude is ``amax_target``."""
    x = rng.standard_normal(shape, dtype=np.float32)
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    x /= np.sqrt(ms + np.float32(1e-6))
    x *= np.float32(amax_target / float(np.max(np.abs(x))))
    return x


def _normal(rng, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _add_outliers(rng, x: np.ndarray, frac: float, lo: float, hi: float) -> int:
    """Replace a random ``frac`` of elements by values with magnitude U[lo, hi]
    and random sign. Returns the number of outliers placed."""
    flat = x.reshape(-1)
    mask = rng.random(flat.shape[0], dtype=np.float32) < np.float32(frac)
    idx = np.nonzero(mask)[0]
    mag = rng.uniform(lo, hi, size=idx.shape[0]).astype(np.float32)
    sign = np.where(rng.random(idx.shape[0]) < 0.5, np.float32(-1), np.float32(1))
    flat[idx] = mag * sign
    return int(idx.shape[0])


def geometric_slopes(num_heads: int, lo_exp: float = -8.0, hi_exp: float = -1.0) -> np.ndarray:
    """Per-head bias slopes geometric in [2^lo_exp, 2^hi_exp]: head 0 gets
    2^hi_exp, the last head 2^lo_exp. Computed in float64, rounded to float32."""
    if num_heads == 1:
        return np.array([2.0 ** hi_exp], dtype=np.float32)
    e = hi_exp + (lo_exp - hi_exp) * np.arange(num_heads, dtype=np.float64) / (num_heads - 1)
    return np.exp2(e).astype(np.float32)


def paged_layout(rng: np.random.Generator, seq_lens, page_size: int = PAGE_SIZE,
                 spare_frac: float = 0.25, min_pool: int = 0):
    """Random page assignment.

    Returns (block_table int32 [B, max_pages], num_pages, slot_mapping int64
    over all tokens in sequence-major order, seq_of_token, pos_of_token).
    Block-table entries past a sequence's last page point at the last pool
    page, which is always a spare (never assigned), so it stays poisoned.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    pages = (seq_lens + page_size - 1) // page_size
    used = int(pages.sum())
    num_pages = max(int(math.ceil(used * (1.0 + spare_frac))), used + 1, min_pool)
    perm = rng.permutation(num_pages - 1).astype(np.int64)  # last page: spare
    max_pages = max(int(pages.max()) if len(pages) else 0, 1)
    bt = np.full((len(seq_lens), max_pages), num_pages - 1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += int(n)
    seq_of = np.repeat(np.arange(len(seq_lens), dtype=np.int64), seq_lens)
    starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]]) if len(seq_lens) else np.zeros(0, np.int64)
    pos_of = np.arange(int(seq_lens.sum()), dtype=np.int64) - np.repeat(starts, seq_lens)
    slot = bt[seq_of, pos_of // page_size].astype(np.int64) * page_size + pos_of % page_size
    return bt, num_pages, slot, seq_of, pos_of


@dataclass
class AttnCase:
    """One e4m3 paged-attention workload (decode when every q_len is 1)."""
    name: str
    seed: int
    seq_lens: np.ndarray          # int32 [B], KV length including the new tokens
    q_lens: np.ndarray            # int32 [B]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    block_table: np.ndarray       # int32 [B, max_pages]
    slot_mapping: np.ndarray      # int64 [T]
    seq_of_token: np.ndarray      # int64 [T]
    pos_of_token: np.ndarray      # int64 [T]
    q: torch.Tensor               # bf16 [sum(q_lens), Hq, D]
    k: torch.Tensor               # bf16 [T, Hkv, D], tokens sequence-major
    v: torch.Tensor               # bf16 [T, Hkv, D]
    store_batches: List[np.ndarray]  # token indices per store call, in order
    window: int = 0
    slopes: Optional[np.ndarray] = None   # float32 [Hq] or None
    rel: Optional[np.ndarray] = None      # learned relative-bias table, float32 [Hq, E] (bf16 values) or None
    softmax_scale: float = 1.0
    fixed_scales: Optional[dict] = None   # {'q','k','v'} floats, or None -> calibrate
    v_scale_override: Optional[float] = None  # fixed v_scale while k/q are calibrated
    notes: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.seq_lens))

    @property
    def cu_q_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    def q_positions(self) -> np.ndarray:
        """Absolute position of every query row (new tokens sit at the end)."""
        out = []
        for L, lq in zip(self.seq_lens, self.q_lens):
            out.append(np.arange(L - lq, L, dtype=np.int64))
        return np.concatenate(out) if out else np.zeros(0, np.int64)


def rel_bias_table(rng, num_heads: int, extent: int) -> np.ndarray:
    """A learned-looking relative-bias table [num_heads, extent], bf16 values:
    a per-head decay -a_h * log(1 + d) in the distance d (a_h geometric in
    [0.25, 2]) plus N(0, 0.25^2) noise, so that near keys weigh more and the
    rows are not smooth."""
    a = np.geomspace(0.25, 2.0, num_heads)[:, None]
    d = np.arange(extent)[None, :]
    t = -a * np.log1p(d) + 0.25 * rng.standard_normal((num_heads, extent))
    return bf16(t.astype(np.float32)).float().numpy()


def make_attn_case(name: str, seed: int, seq_lens, q_lens, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, *, qk_dist: str = "normal",
                   v_std: float = 1.0, v_outlier_frac: float = 0.0,
                   v_outlier_range=(448.0, 1272.0), window: int = 0,
                   slopes: Optional[np.ndarray] = None, fixed_scales: Optional[dict] = None,
                   v_scale_override: Optional[float] = None, spare_frac: float = 0.25,
                   min_pool: int = 0, split_store_at_new: bool = True,
                   softmax_scale: Optional[float] = None, rel_extent: int = 0,
                   v_mean: float = 0.0) -> AttnCase:
    """Draw Q, K, V and a random page layout.

    qk_dist: "normal" for N(0,1), "rms20" for per-row RMS-normed N(0,1) scaled
    so the tensor's amax is 20. V is N(0, v_std^2) with an optional fraction of
    outliers whose magnitude is uniform in v_outlier_range. rel_extent > 0
    adds a learned relative-bias table (see rel_bias_table), drawn after
    everything else so the other draws do not depend on it.
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    T = int(seq_lens.sum())
    nq = int(q_lens.sum())
    if qk_dist == "normal":
        q = _normal(rng, (nq, num_q_heads, head_dim), 1.0)
        k = _normal(rng, (T, num_kv_heads, head_dim), 1.0)
    elif qk_dist == "rms20":
        q = _rms_normed(rng, (nq, num_q_heads, head_dim), 20.0)
        k = _rms_normed(rng, (T, num_kv_heads, head_dim), 20.0)
    else:
        raise ValueError(qk_dist)
    v = _normal(rng, (T, num_kv_heads, head_dim), v_std)
    if v_mean:
        v = v + np.float32(v_mean)
    n_out = _add_outliers(rng, v, v_outlier_frac, *v_outlier_range) if v_outlier_frac > 0 else 0
    bt, num_pages, slot, seq_of, pos_of = paged_layout(rng, seq_lens, PAGE_SIZE, spare_frac, min_pool)
    # store order: tokens already cached first, then the new (query) tokens
    new_start = np.repeat(seq_lens - q_lens, seq_lens).astype(np.int64)
    is_new = pos_of >= new_start
    if split_store_at_new:
        batches = [np.nonzero(~is_new)[0], np.nonzero(is_new)[0]]
    else:
        batches = [np.arange(T, dtype=np.int64)]
    batches = [b for b in batches if b.size]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    rel = rel_bias_table(rng, num_q_heads, rel_extent) if rel_extent > 0 else None
    return AttnCase(
        name=name, seed=seed, seq_lens=seq_lens, q_lens=q_lens, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=PAGE_SIZE,
        num_pages=num_pages, block_table=bt, slot_mapping=slot, seq_of_token=seq_of,
        pos_of_token=pos_of, q=bf16(q), k=bf16(k), v=bf16(v), store_batches=batches,
        window=window, slopes=slopes, rel=rel, softmax_scale=float(softmax_scale),
        fixed_scales=fixed_scales, v_scale_override=v_scale_override,
        notes={"v_outliers": n_out},
    )


# --------------------------------------------------------------------------
# The five workloads the path is measured and parity-tested on.
# --------------------------------------------------------------------------

def config_tiny_decode() -> AttnCase:
    """2 sequences x 256 cached tokens, plus one decode token each (L = 257);
    8 query / 2 KV heads, head_dim 64, unit scales, N(0,1) data, seed 0.
    The pool holds 64 pages in random order; unused pages stay poisoned."""
    return make_attn_case("tiny_decode", 0, [257, 257], [1, 1], 8, 2, 64,
                          fixed_scales={"q": 1.0, "k": 1.0, "v": 1.0}, min_pool=64)


def config_batched_decode(seed: int = 1) -> AttnCase:
    """Batch 64 x 8,192-token context, 32/4 heads, head_dim 128. Q and K are
    RMS-normed with amax 20; V has std 8 and 0.1% outliers in [448, 1272].
    v_scale is fixed at 3.0; q/k scales come from amax calibration."""
    return make_attn_case("batched_decode", seed, [8192] * 64, [1] * 64, 32, 4, 128,
                          qk_dist="rms20", v_std=8.0, v_outlier_frac=1e-3,
                          v_scale_override=3.0, split_store_at_new=False)


def config_long_context(window: int = 0, seed: int = 2) -> AttnCase:
    """Batch 4 x 131,072-token context, 32/4 heads, head_dim 128, the batched
    decode generators; all scales calibrated. window=512 gives the sliding
    window variant over the last 512 tokens."""
    return make_attn_case("long_context" + ("_w%d" % window if window else ""), seed,
                          [131072] * 4, [1] * 4, 32, 4, 128, qk_dist="rms20", v_std=8.0,
                          v_outlier_frac=1e-3, window=window, split_store_at_new=False)


def config_chunked_prefill(seed: int = 3, cached: int = 32768, new: int = 2048,
                           batch: int = 4) -> AttnCase:
    """4 sequences x 2,048 new tokens, causal over 32,768 cached + new tokens,
    32/4 heads, head_dim 128, N(0,1) Q/K/V, calibrated scales, per-head bias
    slopes geometric in [2^-8, 2^-1]."""
    L = cached + new
    return make_attn_case("chunked_prefill", seed, [L] * batch, [new] * batch, 32, 4, 128,
                          slopes=geometric_slopes(32))


# --------------------------------------------------------------------------
# Shapes of the vLLM PR 54705 evidence document, "Tier 1: kernel
# performance": the model there has 8 KV heads of head_dim 128 (so 2 per rank
# at TP4 and 8 at TP1), sliding-window layers of 512 tokens and a learned
# relative bias (extent 128 in the sliding-window tests). Query heads are not
# given; these take a GQA group of 8, as the other workloads.
# --------------------------------------------------------------------------

def config_single_stream_decode(seed: int = 7) -> AttnCase:
    """One sequence decoding over 65,536 cached tokens with a rank's TP4 share
    (decode_kv65536_b1_tp4): 16 query / 2 KV heads, head_dim 128, the batched
    decode generators, calibrated scales."""
    return make_attn_case("single_stream_decode", seed, [65536], [1], 16, 2, 128, qk_dist="rms20",
                          v_std=8.0, v_outlier_frac=1e-3, split_store_at_new=False)


def config_local_prefill(seed: int = 8) -> AttnCase:
    """A sliding-window (local) prefill of 8,192 new tokens on TP1 shapes
    (local_prefill_q8192_tp1): 64 query / 8 KV heads, head_dim 128, window
    512, a learned relative-bias table of extent 128, N(0,1) Q/K/V,
    calibrated scales. The sequence has no earlier tokens."""
    return make_attn_case("local_prefill", seed, [8192], [8192], 64, 8, 128, window=512,
                          rel_extent=128)


def write_path_tokens(seed: int, n: int, num_kv_heads: int, head_dim: int = 128):
    """K/V tokens of the write-path sweep ("Tier 1": 33, 2,048 and 16,384
    tokens per call, two head configurations): n tokens of the batched-decode
    value distributions, written to pages of a fresh pool in random order.
    Returns (k, v, slot_mapping, num_pages)."""
    c = make_attn_case("write_path", seed, [n], [1], num_kv_heads, num_kv_heads, head_dim,
                       qk_dist="rms20", v_std=8.0, v_outlier_frac=1e-3, split_store_at_new=False)
    return c.k, c.v, c.slot_mapping, c.num_pages


@dataclass
class MlaCase:
    """NVFP4 MLA latent-cache decode workload."""
    name: str
    seed: int
    seq_lens: np.ndarray      # int32 [B]
    num_q_heads: int
    latent_dim: int           # 512
    rope_dim: int             # 64
    page_size: int
    num_pages: int
    block_table: np.ndarray   # int32 [B, max_pages]
    slot_mapping: np.ndarray  # int64 [T]
    seq_of_token: np.ndarray
    pos_of_token: np.ndarray
    q: torch.Tensor           # bf16 [B, Hq, latent+rope]
    kv: torch.Tensor          # bf16 [T, latent+rope]
    layer_std: float
    rope_scale: float = 1.0
    softmax_scale: float = 1.0
    q_lens: Optional[np.ndarray] = None   # prefill: new tokens per sequence; q is [sum, Hq, D]

    @property
    def batch(self) -> int:
        return int(len(self.seq_lens))

    @property
    def cu_q_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0


def mla_layer_stds(seed: int = 4, n_layers: int = 4) -> List[float]:
    """Per-layer latent std: the two ends of [0.05, 4] plus uniform draws."""
    rng = np.random.default_rng(seed)
    draws = rng.uniform(0.05, 4.0, size=max(n_layers - 2, 0))
    return [0.05, 4.0] + [float(x) for x in draws]


def make_mla_case(name: str, seed: int, seq_lens, num_q_heads: int = 16,
                  layer_std: float = 1.0, latent_dim: int = 512, rope_dim: int = 64,
                  spare_frac: float = 0.25, rope_scale: float = 1.0) -> MlaCase:
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    T = int(seq_lens.sum())
    dq = latent_dim + rope_dim
    q = _normal(rng, (len(seq_lens), num_q_heads, dq), 1.0)
    kv = _normal(rng, (T, dq), layer_std)
    bt, num_pages, slot, seq_of, pos_of = paged_layout(rng, seq_lens, PAGE_SIZE, spare_frac)
    return MlaCase(name=name, seed=seed, seq_lens=seq_lens, num_q_heads=num_q_heads,
                   latent_dim=latent_dim, rope_dim=rope_dim, page_size=PAGE_SIZE,
                   num_pages=num_pages, block_table=bt, slot_mapping=slot,
                   seq_of_token=seq_of, pos_of_token=pos_of, q=bf16(q), kv=bf16(kv),
                   layer_std=float(layer_std), rope_scale=float(rope_scale),
                   softmax_scale=1.0 / math.sqrt(dq))


def config_nvfp4_mla(layer: int = 0, seed: int = 4, batch: int = 32,
                     context: int = 16384) -> MlaCase:
    """Batch 32 x 16,384-token context, 16 query heads sharing one latent head
    (512 latent + 64 RoPE dims), latents N(0, std^2) with the layer's std."""
    std = mla_layer_stds(seed)[layer]
    return make_mla_case("nvfp4_mla_l%d" % layer, seed * 10 + layer, [context] * batch,
                         16, layer_std=std)


def config_nvfp4_mla_prefill(seed: int = 5, batch: int = 4, context: int = 16384,
                             new: int = 1024, layer_std: float = 1.0) -> MlaCase:
    """Chunked prefill over the NVFP4 latent cache: 4 sequences whose last
    1,024 of 16,384 tokens are new, 16 query heads, N(0,1) queries."""
    c = make_mla_case("nvfp4_mla_prefill", seed, [context] * batch, 16, layer_std=layer_std)
    rng = np.random.default_rng(seed + 1000)
    c.q_lens = np.full(batch, new, dtype=np.int32)
    c.q = bf16(_normal(rng, (batch * new, c.num_q_heads, c.latent_dim + c.rope_dim), 1.0))
    return c


CONFIGS = {
    "single_stream_decode": config_single_stream_decode,
    "local_prefill": config_local_prefill,
    "tiny_decode": config_tiny_decode,
    "batched_decode": config_batched_decode,
    "long_context": config_long_context,
    "chunked_prefill": config_chunked_prefill,
    "nvfp4_mla": config_nvfp4_mla,
    "nvfp4_mla_prefill": config_nvfp4_mla_prefill,
}
