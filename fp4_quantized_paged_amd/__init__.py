"""kvq: quantized-KV-cache attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libkvq.so`` (include/kvq.h). It only
marshals arguments: torch tensors provide device memory and the current HIP
stream, every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

FMT_E4M3 = 1
FMT_NVFP4_MLA368 = 2
PAGE_SIZE = 16
RECORD_BYTES = 368

STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID_ARG", -2: "KVQ_ERR_UNSUPPORTED",
          -3: "KVQ_ERR_BAD_SCALE", -4: "KVQ_ERR_WORKSPACE", -5: "KVQ_ERR_HIP",
          -6: "KVQ_ERR_SCRATCH_LIMIT"}

NOALLOC_SCRATCH_BYTES = 16 << 20   # KVQ_NOALLOC_SCRATCH_BYTES of include/kvq.h


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), status_str(status)))


class CacheDesc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class AttnParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("rel_extent", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("q_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("alibi_slopes", ctypes.c_void_p), ("rel_bias", ctypes.c_void_p),
                ("flags", ctypes.c_uint32)]

FLAG_PREFILL_FP8_P = 1
FLAG_PREFILL_FP8_P2 = 2


_lib = None
ABI_VERSION = 7   # KVQ_ABI_VERSION of include/kvq.h

_SIGNATURES = {
    "kvq_abi_version": (ctypes.c_int, []),
    "kvq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_store": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_float, ctypes.c_float, ctypes.c_void_p]),
    "kvq_store_nvfp4_static": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_float, ctypes.c_void_p]),
    "kvq_calibrate_amax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "kvq_scale_from_amax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "kvq_band_counts": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "kvq_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc), ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.POINTER(AttnParams)]),
    "kvq_paged_attn_decode": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(AttnParams), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvq_paged_attn_decode_append": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                    ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.POINTER(AttnParams), ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvq_paged_attn_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.POINTER(AttnParams), ctypes.c_void_p,
                                                     ctypes.c_void_p]),
    "kvq_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc), ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.POINTER(AttnParams)]),
    "kvq_paged_attn_prefill": (ctypes.c_int, [ctypes.POINTER(CacheDesc), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(AttnParams), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """Load libkvq.so once. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so not found at %s: build it with "
                               "`python -m fp4_quantized_paged_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        handle.kvq_abi_version.restype = ctypes.c_int
        handle.kvq_abi_version.argtypes = []
        if handle.kvq_abi_version() != ABI_VERSION:
            raise RuntimeError("%s has ABI version %d, this binding expects %d: rebuild it"
                               % (LIB_PATH, handle.kvq_abi_version(), ABI_VERSION))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    try:
        return lib().kvq_status_str(int(status)).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "?"


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KvqError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("kvq needs device tensors")


def _check_rows(name: str, t: torch.Tensor, inner: tuple) -> None:
    """t is bf16 [T, *inner] with the inner dims dense (token stride free)."""
    if t.dtype != torch.bfloat16 or tuple(t.shape[1:]) != tuple(inner):
        raise ValueError("%s must be bf16 [T, %s], got %s %s" % (name, ", ".join(map(str, inner)),
                                                                 t.dtype, tuple(t.shape)))
    step = 1
    for dim in range(t.dim() - 1, 0, -1):
        if t.shape[dim] > 1 and t.stride(dim) != step:
            raise ValueError("%s: each token's %s elements must be contiguous (strides %s)"
                             % (name, "x".join(map(str, inner)), tuple(t.stride())))
        step *= t.shape[dim]


def _head_dims(cache) -> tuple:
    d = cache.desc
    return (576, 512) if d.format == FMT_NVFP4_MLA368 else (d.head_dim, d.head_dim)


def _check_decode_args(cache, q, block_table, seq_lens) -> None:
    dqk, _ = _head_dims(cache)
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_contiguous() or q.shape[2] != dqk:
        raise ValueError("q must be contiguous bf16 [B, Hq, %d], got %s %s" % (dqk, q.dtype, tuple(q.shape)))
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, pages] with unit inner stride")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 vector")
    if seq_lens.shape[0] != q.shape[0] or block_table.shape[0] < q.shape[0]:
        raise ValueError("q, seq_lens and block_table disagree on the number of sequences")


def _check_out(out: torch.Tensor, shape: tuple) -> None:
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError("out must be contiguous bf16 %s, got %s %s" % (shape, out.dtype, tuple(out.shape)))


class E4M3Cache:
    """Paged e4m3 K/V pools: K u8 [pages][Hkv][16][D], V u8 [pages][Hkv][D][16]."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int,
                 device="cuda", fill: int = 0x7F):
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.k = torch.full((num_pages, num_kv_heads, PAGE_SIZE, head_dim), fill,
                            dtype=torch.uint8, device=device)
        self.v = torch.full((num_pages, num_kv_heads, head_dim, PAGE_SIZE), fill,
                            dtype=torch.uint8, device=device)

    @property
    def desc(self) -> CacheDesc:
        return CacheDesc(FMT_E4M3, PAGE_SIZE, self.num_kv_heads, self.head_dim,
                         self.num_pages, self.k.data_ptr(), self.v.data_ptr())


class Nvfp4Cache:
    """Paged NVFP4 MLA records: u8 [pages][16][368]."""

    def __init__(self, num_pages: int, device="cuda", fill: int = 0x7F):
        self.num_pages = num_pages
        self.records = torch.full((num_pages, PAGE_SIZE, RECORD_BYTES), fill, dtype=torch.uint8,
                                  device=device)

    @property
    def desc(self) -> CacheDesc:
        return CacheDesc(FMT_NVFP4_MLA368, PAGE_SIZE, 1, 576, self.num_pages,
                         self.records.data_ptr(), None)


def store(cache, k: torch.Tensor, v: Optional[torch.Tensor], slot_mapping: torch.Tensor,
          k_scale: float, v_scale: float = 1.0) -> None:
    """kvq_store. E4M3: k, v bf16 [T, Hkv, D]; NVFP4: k bf16 [T, 576], v None
    and k_scale the RoPE scale. slot_mapping int64 [T] (negative: skip)."""
    _need_cuda(k, v, slot_mapping)
    d = cache.desc
    T = k.shape[0]
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,) or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 [T] vector")
    if d.format == FMT_NVFP4_MLA368:
        _check_rows("k", k, (576,))
        if v is not None:
            raise ValueError("the NVFP4 record store takes no v")
    else:
        _check_rows("k", k, (d.num_kv_heads, d.head_dim))
        if v is None or v.shape[0] != T:
            raise ValueError("v must hold the same tokens as k")
        _check_rows("v", v, (d.num_kv_heads, d.head_dim))
    st = lib().kvq_store(ctypes.byref(d), _ptr(k), k.stride(0), _ptr(v),
                         v.stride(0) if v is not None else 0, _ptr(slot_mapping), T,
                         float(k_scale), float(v_scale), _stream())
    _check(st, "kvq_store")


def store_nvfp4_static(cache, x: torch.Tensor, slot_mapping: torch.Tensor, rope_scale: float,
                       outer_scale: float) -> None:
    """kvq_store_nvfp4_static: NVFP4 records with one static outer scale for
    every token. x bf16 [T, 576], slot_mapping int64 [T]."""
    _need_cuda(x, slot_mapping)
    _check_rows("x", x, (576,))
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (x.shape[0],) or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 [T] vector")
    st = lib().kvq_store_nvfp4_static(ctypes.byref(cache.desc), _ptr(x), x.stride(0), _ptr(slot_mapping),
                                      x.shape[0], float(rope_scale), float(outer_scale), _stream())
    _check(st, "kvq_store_nvfp4_static")


def calibrate_amax(x: torch.Tensor, slot_mapping: Optional[torch.Tensor] = None,
                   amax: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None):
    """kvq_calibrate_amax over the rows of x (bf16, first dim = rows, the rest
    flattened). Returns (amax, scale) as 1-element device fp32 tensors; pass
    ``amax`` to keep a running value."""
    _need_cuda(x, slot_mapping)
    assert x.dtype == torch.bfloat16
    rows = x.shape[0]
    row_len = 1
    for n in x.shape[1:]:
        row_len *= int(n)
    x2 = x.reshape(rows, row_len)
    if amax is None:
        amax = torch.zeros(1, dtype=torch.float32, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    st = lib().kvq_calibrate_amax(_ptr(x2), rows, row_len, x2.stride(0) if rows else row_len,
                                  _ptr(slot_mapping), _ptr(amax), _ptr(scale), _stream())
    _check(st, "kvq_calibrate_amax")
    return amax, scale


SCALE_AMAX_448, SCALE_CEIL_BF16, SCALE_SAFETY_1P3 = 0, 1, 2


def scale_from_amax(amax: torch.Tensor, rule: int, scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvq_scale_from_amax: the scale of a running amax (1-element device fp32)
    under one of the SCALE_* rules, as a 1-element device fp32 tensor."""
    _need_cuda(amax)
    assert amax.dtype == torch.float32
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=amax.device)
    _check(lib().kvq_scale_from_amax(_ptr(amax), int(rule), _ptr(scale), _stream()), "kvq_scale_from_amax")
    return scale


def band_counts(x: torch.Tensor, scale: float, slot_mapping: Optional[torch.Tensor] = None,
                counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvq_band_counts over the rows of x (bf16, first dim = rows): adds the
    (clipped, flushed) counts at ``scale`` to ``counts`` (device int64 [2],
    zeros when not given) and returns it."""
    _need_cuda(x, slot_mapping)
    assert x.dtype == torch.bfloat16
    rows = x.shape[0]
    row_len = 1
    for n in x.shape[1:]:
        row_len *= int(n)
    x2 = x.reshape(rows, row_len)
    if counts is None:
        counts = torch.zeros(2, dtype=torch.int64, device=x.device)
    assert counts.dtype == torch.int64 and counts.numel() == 2 and counts.is_contiguous()
    st = lib().kvq_band_counts(_ptr(x2), rows, row_len, x2.stride(0) if rows else row_len,
                               _ptr(slot_mapping), float(scale), _ptr(counts), _stream())
    _check(st, "kvq_band_counts")
    return counts


def _params(num_q_heads, softmax_scale, q_scale, k_scale, v_scale, window, slopes, num_splits,
            rel_bias=None, flags=0):
    if rel_bias is not None:
        assert rel_bias.dtype == torch.bfloat16 and rel_bias.is_contiguous() and rel_bias.dim() == 2
        assert rel_bias.shape[0] == num_q_heads
    extent = 0 if rel_bias is None else int(rel_bias.shape[1])
    return AttnParams(int(num_q_heads), int(window), int(num_splits), extent, float(softmax_scale),
                      float(q_scale), float(k_scale), float(v_scale), _ptr(slopes), _ptr(rel_bias),
                      int(flags))


def decode_workspace_bytes(cache, num_seqs: int, max_seq_len: int, num_q_heads: int,
                           window: int = 0, num_splits: int = 0, softmax_scale: float = 1.0) -> int:
    d = cache.desc
    p = _params(num_q_heads, softmax_scale, 1.0, 1.0, 1.0, window, None, num_splits)
    return int(lib().kvq_decode_workspace_bytes(ctypes.byref(d), int(num_seqs), int(max_seq_len),
                                                ctypes.byref(p)))


def decode(cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
           max_seq_len: int, softmax_scale: float, q_scale: float = 1.0, k_scale: float = 1.0,
           v_scale: float = 1.0, window: int = 0, slopes: Optional[torch.Tensor] = None,
           num_splits: int = 0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None,
           rel_bias: Optional[torch.Tensor] = None, k_new: Optional[torch.Tensor] = None,
           v_new: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvq_paged_attn_decode. q bf16 [B, Hq, Dqk] -> out bf16 [B, Hq, Dv].
    rel_bias: learned relative-bias table, bf16 [Hq, extent]. k_new, v_new
    (bf16 [B, Hkv, D], both or neither): the current tokens' K/V, stored at
    position seq_lens[b] - 1 with k_scale / v_scale in the same launch
    (kvq_paged_attn_decode_append)."""
    _need_cuda(q, block_table, seq_lens, slopes, rel_bias, k_new, v_new)
    append = k_new is not None or v_new is not None
    if append:
        assert k_new is not None and v_new is not None
        d0 = cache.desc
        for t in (k_new, v_new):
            if (t.dtype != torch.bfloat16 or not t.is_contiguous()
                    or tuple(t.shape) != (q.shape[0], d0.num_kv_heads, d0.head_dim)):
                raise ValueError("k_new / v_new must be contiguous bf16 [B, Hkv, D]")
    _need_cuda(out)
    _check_decode_args(cache, q, block_table, seq_lens)
    B, Hq, _ = q.shape
    d = cache.desc
    dv = _head_dims(cache)[1]
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _check_out(out, (B, Hq, dv))
    p = _params(Hq, softmax_scale, q_scale, k_scale, v_scale, window, slopes, num_splits, rel_bias)
    need = int(lib().kvq_decode_workspace_bytes(ctypes.byref(d), B, int(max_seq_len), ctypes.byref(p)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if append:
        st = lib().kvq_paged_attn_decode_append(ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new),
                                                _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
                                                B, int(max_seq_len), ctypes.byref(p), _ptr(out),
                                                _ptr(workspace), ws_bytes, _stream())
        _check(st, "kvq_paged_attn_decode_append")
        return out
    st = lib().kvq_paged_attn_decode(ctypes.byref(d), _ptr(q), _ptr(block_table),
                                     block_table.stride(0), _ptr(seq_lens), B, int(max_seq_len),
                                     ctypes.byref(p), _ptr(out), _ptr(workspace), ws_bytes,
                                     _stream())
    _check(st, "kvq_paged_attn_decode")
    return out


def decode_noalloc(cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                   max_seq_len: int, softmax_scale: float, q_scale: float = 1.0, k_scale: float = 1.0,
                   v_scale: float = 1.0, window: int = 0, slopes: Optional[torch.Tensor] = None,
                   num_splits: int = 0, out: Optional[torch.Tensor] = None,
                   rel_bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvq_paged_attn_decode_noalloc: decode with the split partials in the
    library's static scratch array (no workspace). Pass ``out`` to keep the
    call free of allocations on this side too."""
    _need_cuda(q, block_table, seq_lens, slopes, rel_bias, out)
    _check_decode_args(cache, q, block_table, seq_lens)
    B, Hq, _ = q.shape
    d = cache.desc
    dv = 512 if d.format == FMT_NVFP4_MLA368 else d.head_dim
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _check_out(out, (B, Hq, dv))
    p = _params(Hq, softmax_scale, q_scale, k_scale, v_scale, window, slopes, num_splits, rel_bias)
    st = lib().kvq_paged_attn_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(block_table),
                                             block_table.stride(0), _ptr(seq_lens), B, int(max_seq_len),
                                             ctypes.byref(p), _ptr(out), _stream())
    _check(st, "kvq_paged_attn_decode_noalloc")
    return out


def prefill_workspace_bytes(cache, num_seqs: int, max_seq_len: int, num_q_heads: int,
                            slopes: Optional[torch.Tensor] = None, softmax_scale: float = 1.0) -> int:
    """kvq_prefill_workspace_bytes: bytes of the optional per-block key-norm
    workspace of a slope-bias prefill (0 when it does not apply)."""
    p = _params(num_q_heads, softmax_scale, 1.0, 1.0, 1.0, 0, slopes, 0)
    return int(lib().kvq_prefill_workspace_bytes(ctypes.byref(cache.desc), int(num_seqs), int(max_seq_len),
                                                 ctypes.byref(p)))


def prefill(cache, q: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int,
            block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
            softmax_scale: float, q_scale: float = 1.0, k_scale: float = 1.0,
            v_scale: float = 1.0, window: int = 0, slopes: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, rel_bias: Optional[torch.Tensor] = None,
            fp8_p: bool = False, fp8_p2: bool = False,
            workspace: Optional[torch.Tensor] = None, use_workspace: bool = True) -> torch.Tensor:
    """kvq_paged_attn_prefill. q bf16 [sumQ, Hq, Dqk] -> out bf16 [sumQ, Hq, Dv].
    rel_bias: learned relative-bias table, bf16 [Hq, extent]. fp8_p: the
    single-term e4m3 P speed variant (KVQ_FLAG_PREFILL_FP8_P); fp8_p2: the
    two-term e4m3 P path (KVQ_FLAG_PREFILL_FP8_P2). With slopes, the
    per-block key-norm workspace is used (allocated here when not passed)
    unless use_workspace is False; the output is the same either way."""
    _need_cuda(q, cu_q_lens, block_table, seq_lens, slopes, rel_bias, out, workspace)
    dqk, dv = _head_dims(cache)
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_contiguous() or q.shape[2] != dqk:
        raise ValueError("q must be contiguous bf16 [sumQ, Hq, %d], got %s %s" % (dqk, q.dtype, tuple(q.shape)))
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, pages] with unit inner stride")
    B = int(seq_lens.shape[0])
    if (seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous()
            or cu_q_lens.dtype != torch.int32 or tuple(cu_q_lens.shape) != (B + 1,)
            or not cu_q_lens.is_contiguous() or block_table.shape[0] < B):
        raise ValueError("seq_lens int32 [B], cu_q_lens int32 [B + 1] and block_table [>= B, pages] expected")
    total_q, Hq, D = q.shape
    d = cache.desc
    if out is None:
        out = torch.empty((total_q, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _check_out(out, (total_q, Hq, dv))
    p = _params(Hq, softmax_scale, q_scale, k_scale, v_scale, window, slopes, 0, rel_bias,
                (FLAG_PREFILL_FP8_P if fp8_p else 0) | (FLAG_PREFILL_FP8_P2 if fp8_p2 else 0))
    ws_bytes = 0
    if use_workspace:
        need = int(lib().kvq_prefill_workspace_bytes(ctypes.byref(d), B, int(max_seq_len), ctypes.byref(p)))
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    else:
        workspace = None
    st = lib().kvq_paged_attn_prefill(ctypes.byref(d), _ptr(q), _ptr(cu_q_lens), total_q,
                                      int(max_q_len), _ptr(block_table), block_table.stride(0),
                                      _ptr(seq_lens), int(seq_lens.shape[0]), int(max_seq_len),
                                      ctypes.byref(p), _ptr(out), _ptr(workspace), ws_bytes, _stream())
    _check(st, "kvq_paged_attn_prefill")
    return out
