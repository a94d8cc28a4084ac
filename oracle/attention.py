"""Paged attention over the e4m3 cache, in fp64.

Test infrastructure only (see the package header).

What is computed (vLLM PR 54705, "Purpose" query-quantization and
descale-handling bullets):
  * Q is quantized with the same saturating e4m3 quantizer as the cache, using
    its own per-tensor q_scale;
  * raw scores are dot products of the decoded e4m3 codes; the QK descale is
    folded into the softmax scale, s = raw * (softmax_scale * q_scale * k_scale),
    and only then is the exact bf16 relative bias added;
  * softmax over the attended keys; the V descale multiplies the output, which
    is linear in V.
Readings where the pages are silent:
  * bias(h, i, j) = bf16_RNE(fp32(slope_h) * fp32(-(p_i - j))), a per-head
    linear bias in the query-key distance, added in fp32 after the fold;
  * the learned relative position bias (same page, "Environment": the model
    has one; "Test Plan": relative extents 128 and 1024, and 128 with the
    sliding window) is a bf16 table T[h][0 .. E) indexed by the query-key
    distance: bias(h, i, j) = T[h][min(p_i - j, E - 1)], the last entry
    serving every longer distance. It replaces the slope bias and enters at
    the same place;
  * a query at absolute position p attends keys j <= p; with a sliding window
    W > 0 only keys with p - W < j <= p (the window includes the current
    token); W = 0 means full attention; new queries sit at the end of the
    sequence (position L - Lq + i);
  * GQA: query head h reads KV head h // (Hq / Hkv);
  * a query with no keys (sequence length 0) outputs zeros.
Probabilities are kept exact here (fp64). The kernel's rounding of P is a
performance choice checked against this within tolerance.

Split-KV (vLLM PR 54705 evidence, "Tier 0": online softmax across blocks):
``attend_split`` cuts the key range into chunks, keeps (m, l, o) per chunk and
merges them with o = sum_c e^(m_c - m) o_c / sum_c e^(m_c - m) l_c. It must equal
the unsplit result to rounding.

Pins: tests/test_oracle_attention.py (pure-Python brute force, fold vs explicit
dequantisation, V linearity, split invariance, window reduction, Q = 0 mean,
single key, zero slope, repeated-KV-head GQA equivalence; learned table: the
closed-form softmax of a Q = 0 case with one-hot V, and a table filled with
the slope bias reproducing the slope path).
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_decode, bf16_round
from .kvcache import quantize_e4m3, gather_tokens


def relative_bias(slope: float, q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """bf16-exact bias values [len(q_pos), len(k_pos)] as float64."""
    dist = (np.asarray(q_pos, dtype=np.int64)[:, None] - np.asarray(k_pos, dtype=np.int64)[None, :])
    prod = np.float32(slope) * (-dist).astype(np.float32)
    return bf16_round(prod).astype(np.float64)


def learned_bias(table_h: np.ndarray, q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """Learned relative bias of one head, [len(q_pos), len(k_pos)] float64:
    entry min(p - j, E - 1) of the bf16 row table_h [E] for key j at or before
    the query position p; keys after p (masked anyway) read entry 0."""
    E = len(table_h)
    dist = (np.asarray(q_pos, dtype=np.int64)[:, None] - np.asarray(k_pos, dtype=np.int64)[None, :])
    return np.asarray(table_h, dtype=np.float64)[np.clip(dist, 0, E - 1)]


def _bias(h: int, q_pos, k_pos, slopes, rel):
    """The additive bias of head h, or None (at most one kind is given)."""
    if slopes is not None:
        return relative_bias(float(slopes[h]), q_pos, k_pos)
    if rel is not None:
        return learned_bias(rel[h], q_pos, k_pos)
    return None


def key_mask(q_pos: np.ndarray, L: int, window: int) -> np.ndarray:
    """Boolean [nq, L]: which keys each query attends."""
    j = np.arange(L, dtype=np.int64)[None, :]
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    m = j <= p
    if window > 0:
        m &= j > p - window
    return m


def _softmax_out(s: np.ndarray, mask: np.ndarray, vals: np.ndarray):
    """Masked softmax rows of s [n, L] applied to vals [L, Dv] -> (o, m, l), o
    normalised. Rows without keys give zeros."""
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(mask, np.exp(s - m_safe[:, None]), 0.0)
    l = w.sum(axis=1)
    o = w @ vals
    o = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return o, m, l


def attend_sequence(q_codes_val: np.ndarray, q_pos: np.ndarray, k_val: np.ndarray,
                    v_val: np.ndarray, fold: float, v_scale: float, window: int,
                    slopes, q_chunk: int = 64, rel=None) -> np.ndarray:
    """Attention of one sequence's queries.

    q_codes_val: decoded e4m3 Q [nq, Hq, D]; k_val [L, Hkv, D] and
    v_val [L, Hkv, Dv] decoded e4m3 (unscaled). slopes [Hq] or rel [Hq][E]
    (bf16 values) select the bias. Returns fp64 [nq, Hq, Dv]."""
    nq, Hq, D = q_codes_val.shape
    L, Hkv, Dv = v_val.shape
    grp = Hq // Hkv
    out = np.zeros((nq, Hq, Dv), dtype=np.float64)
    if L == 0 or nq == 0:
        return out
    k_pos = np.arange(L, dtype=np.int64)
    for c0 in range(0, nq, q_chunk):
        c1 = min(nq, c0 + q_chunk)
        qp = q_pos[c0:c1]
        mask = key_mask(qp, L, window)
        for h in range(Hq):
            g = h // grp
            raw = q_codes_val[c0:c1, h, :] @ k_val[:, g, :].T
            s = raw * fold
            bias = _bias(h, qp, k_pos, slopes, rel)
            if bias is not None:
                s = s + bias
            o, _, _ = _softmax_out(s, mask, v_val[:, g, :])
            out[c0:c1, h, :] = o * v_scale
    return out


def attend_split(q_codes_val, q_pos, k_val, v_val, fold, v_scale, window, slopes,
                 chunk: int, rel=None) -> np.ndarray:
    """Same as attend_sequence, but over key chunks of ``chunk`` keys merged
    with the online-softmax combine."""
    nq, Hq, D = q_codes_val.shape
    L, Hkv, Dv = v_val.shape
    grp = Hq // Hkv
    out = np.zeros((nq, Hq, Dv), dtype=np.float64)
    if L == 0 or nq == 0:
        return out
    k_pos = np.arange(L, dtype=np.int64)
    mask = key_mask(q_pos, L, window)
    for h in range(Hq):
        g = h // grp
        s = (q_codes_val[:, h, :] @ k_val[:, g, :].T) * fold
        bias = _bias(h, q_pos, k_pos, slopes, rel)
        if bias is not None:
            s = s + bias
        parts = []
        for j0 in range(0, L, chunk):
            j1 = min(L, j0 + chunk)
            o, m, l = _softmax_out(s[:, j0:j1], mask[:, j0:j1], v_val[j0:j1, g, :])
            parts.append((o * l[:, None], m, l))        # unnormalised partial
        m_all = np.max(np.stack([p[1] for p in parts]), axis=0)
        m_safe = np.where(np.isfinite(m_all), m_all, 0.0)
        num = np.zeros((nq, Dv))
        den = np.zeros(nq)
        for o_u, m_c, l_c in parts:
            wgt = np.where(np.isfinite(m_c), np.exp(np.where(np.isfinite(m_c), m_c, 0.0) - m_safe), 0.0)
            num += wgt[:, None] * o_u
            den += wgt * l_c
        out[:, h, :] = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0) * v_scale
    return out


def quantize_q(q: np.ndarray, q_scale: float) -> np.ndarray:
    """bf16 Q (as float32) -> decoded e4m3 values (unscaled), float64."""
    return e4m3_decode(quantize_e4m3(q, q_scale))


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_table: np.ndarray, seq_lens: np.ndarray, softmax_scale: float,
                 q_scale: float, k_scale: float, v_scale: float, window: int = 0,
                 slopes=None, seqs=None, rel=None) -> np.ndarray:
    """One query per sequence at position L-1. q: [B, Hq, D] float32 (bf16
    values). Returns fp64 [B, Hq, Dv] (rows of sequences not in ``seqs`` are
    left zero)."""
    B, Hq, D = q.shape
    Dv = v_cache.shape[2]
    out = np.zeros((B, Hq, Dv), dtype=np.float64)
    fold = float(softmax_scale) * float(q_scale) * float(k_scale)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        if L == 0:
            continue
        kc, vc = gather_tokens(k_cache, v_cache, block_table[b], L)
        qv = quantize_q(q[b:b + 1], q_scale)
        out[b] = attend_sequence(qv, np.array([L - 1]), e4m3_decode(kc), e4m3_decode(vc),
                                 fold, v_scale, window, slopes, rel=rel)[0]
    return out


def paged_prefill(q: np.ndarray, cu_q_lens: np.ndarray, k_cache: np.ndarray,
                  v_cache: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                  softmax_scale: float, q_scale: float, k_scale: float, v_scale: float,
                  window: int = 0, slopes=None, rows=None, rel=None) -> np.ndarray:
    """Chunked prefill: the new queries of sequence b are rows
    cu_q_lens[b]..cu_q_lens[b+1]-1 of q [sumQ, Hq, D] at positions
    L - Lq + i. ``rows`` optionally restricts the computed query rows
    (global row indices); other rows stay zero."""
    nrows, Hq, D = q.shape
    Dv = v_cache.shape[2]
    out = np.zeros((nrows, Hq, Dv), dtype=np.float64)
    fold = float(softmax_scale) * float(q_scale) * float(k_scale)
    want = None if rows is None else np.zeros(nrows, dtype=bool)
    if want is not None:
        want[np.asarray(rows, dtype=np.int64)] = True
    for b in range(len(seq_lens)):
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        L = int(seq_lens[b])
        idx = np.arange(r0, r1)
        if want is not None:
            idx = idx[want[r0:r1]]
        if idx.size == 0 or L == 0:
            continue
        lq = r1 - r0
        pos = L - lq + (idx - r0)
        kc, vc = gather_tokens(k_cache, v_cache, block_table[b], L)
        qv = quantize_q(q[idx], q_scale)
        out[idx] = attend_sequence(qv, pos, e4m3_decode(kc), e4m3_decode(vc), fold,
                                   v_scale, window, slopes, rel=rel)
    return out


def brute_force(q_vals, q_pos, k_vals, v_vals, softmax_scale, window, slopes, rel=None):
    """Pure-Python triple loop over already-dequantized values (no numpy
    reductions), for tiny inputs. q_vals [nq][Hq][D], k_vals [L][Hkv][D],
    v_vals [L][Hkv][Dv] as nested lists of floats; rel: per-head lists of
    table values. Returns nested lists."""
    import math
    nq, Hq = len(q_vals), len(q_vals[0])
    L, Hkv = len(k_vals), len(k_vals[0])
    D, Dv = len(q_vals[0][0]), len(v_vals[0][0])
    grp = Hq // Hkv
    out = []
    for i in range(nq):
        p = int(q_pos[i])
        row = []
        for h in range(Hq):
            g = h // grp
            keys = [j for j in range(L) if j <= p and (window <= 0 or j > p - window)]
            scores = []
            for j in keys:
                acc = 0.0
                for d in range(D):
                    acc += q_vals[i][h][d] * k_vals[j][g][d]
                s = acc * softmax_scale
                if slopes is not None:
                    s += float(bf16_round(np.float32(slopes[h]) * np.float32(-(p - j))))
                if rel is not None:
                    s += float(rel[h][min(p - j, len(rel[h]) - 1)])
                scores.append(s)
            if not keys:
                row.append([0.0] * Dv)
                continue
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            row.append([sum(ws[t] * v_vals[j][g][d] for t, j in enumerate(keys)) / tot
                        for d in range(Dv)])
        out.append(row)
    return out
