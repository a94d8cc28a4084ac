"""Helpers shared by the GPU parity tests: move a seeded workload to the
device, run the oracle on the same seeded inputs, and compare.

The two sides never exchange data: both start from the arrays the workload
generator produced; the oracle runs on the CPU, the HIP path through the
C ABI."""
from __future__ import annotations

import numpy as np
import torch

import fp4_quantized_paged_amd as kvq
from oracle.kvcache import new_cache, store_e4m3, calibrate_amax

# Attention tolerance: rel-L2 <= 5e-3 and |o - ref| <= 2e-2 * max(1, |ref|)
# elementwise (the plain 2e-2 bound where |ref| <= 1; bf16 output rounding
# alone is 2^-9 |ref|, so a fixed absolute bound cannot hold for large outputs).
REL_L2 = 5e-3
ABS_TOL = 2e-2


def check_attention(got: torch.Tensor, ref: np.ndarray, label: str = "") -> dict:
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), label + ": non-finite output"
    err = np.abs(g - ref)
    bound = ABS_TOL * np.maximum(1.0, np.abs(ref))
    worst = float(np.max(err / bound)) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref) / denom) if denom > 0 else float(np.linalg.norm(g))
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "rel_l2": rel, "worst_ratio": worst}
    assert worst <= 1.0, "%s: elementwise bound exceeded %s" % (label, stats)
    assert rel <= REL_L2, "%s: rel-L2 exceeded %s" % (label, stats)
    return stats


class DeviceCase:
    """A workload's tensors on the GPU plus its e4m3 cache."""

    def __init__(self, case, device="cuda", fill=0x7F):
        self.case = case
        self.cache = kvq.E4M3Cache(case.num_pages, case.num_kv_heads, case.head_dim, device, fill)
        self.k = case.k.to(device)
        self.v = case.v.to(device)
        self.q = case.q.to(device)
        self.slot = torch.from_numpy(case.slot_mapping).to(device)
        self.block_table = torch.from_numpy(case.block_table).to(device)
        self.seq_lens = torch.from_numpy(case.seq_lens).to(device)
        self.cu_q_lens = torch.from_numpy(case.cu_q_lens).to(device)
        self.slopes = None if case.slopes is None else torch.from_numpy(case.slopes).to(device)
        self.rel = None if case.rel is None else torch.from_numpy(case.rel).to(torch.bfloat16).to(device)

    def calibrate(self):
        """GPU amax/448 scales (read back once, as a caller would)."""
        c = self.case
        out = {}
        for name, x in (("k", self.k), ("v", self.v), ("q", self.q)):
            _, s = kvq.calibrate_amax(x)
            out[name] = float(s.item())
        if c.fixed_scales is not None:
            out = dict(c.fixed_scales)
        if c.v_scale_override is not None:
            out["v"] = float(c.v_scale_override)
        return out

    def store_all(self, scales):
        for idx in self.case.store_batches:
            i = torch.from_numpy(idx).to(self.k.device)
            kvq.store(self.cache, self.k[i].contiguous(), self.v[i].contiguous(), self.slot[i],
                      scales["k"], scales["v"])

    def decode(self, scales, **kw):
        c = self.case
        return kvq.decode(self.cache, self.q, self.block_table, self.seq_lens, c.max_seq_len,
                          c.softmax_scale, scales["q"], scales["k"], scales["v"], c.window,
                          self.slopes, rel_bias=self.rel, **kw)

    def prefill(self, scales, **kw):
        c = self.case
        return kvq.prefill(self.cache, self.q, self.cu_q_lens, c.max_q_len, self.block_table,
                           self.seq_lens, c.max_seq_len, c.softmax_scale, scales["q"],
                           scales["k"], scales["v"], c.window, self.slopes, rel_bias=self.rel, **kw)


def oracle_scales(case):
    """The oracle's own amax/448 scales from the seeded inputs."""
    if case.fixed_scales is not None:
        s = dict(case.fixed_scales)
    else:
        s = {}
        for name, x in (("k", case.k), ("v", case.v), ("q", case.q)):
            _, sc = calibrate_amax(x.float().numpy())
            s[name] = float(sc)
    if case.v_scale_override is not None:
        s["v"] = float(case.v_scale_override)
    return s


def oracle_cache(case, scales, tokens=None):
    """Oracle K/V pools after all store batches (optionally only ``tokens``)."""
    kc, vc = new_cache(case.num_pages, case.num_kv_heads, case.page_size, case.head_dim)
    k = case.k.float().numpy()
    v = case.v.float().numpy()
    slot = case.slot_mapping
    for idx in case.store_batches:
        if tokens is not None:
            idx = np.intersect1d(idx, tokens)
        store_e4m3(kc, vc, k[idx], v[idx], slot[idx], scales["k"], scales["v"])
    return kc, vc


def seq_tokens(case, seqs):
    """Global token indices of the given sequences."""
    starts = np.concatenate([[0], np.cumsum(case.seq_lens)])
    return np.concatenate([np.arange(starts[b], starts[b + 1]) for b in seqs])
