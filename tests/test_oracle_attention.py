"""Pins for the oracle's attention: brute force, algebraic identities the pages
rely on (fold, V linearity), online-softmax split invariance, window and
degenerate cases."""
import math

import numpy as np
import pytest

from oracle.codecs import e4m3_decode, bf16_round
from oracle.kvcache import quantize_e4m3, new_cache, store_e4m3, gather_tokens
from oracle.attention import (attend_sequence, attend_split, brute_force, paged_decode,
                              paged_prefill, quantize_q, relative_bias, learned_bias)
from workloads import make_attn_case, geometric_slopes


def tiny(seed=0, L=19, Hq=4, Hkv=2, D=8, nq=3, v_std=1.0):
    rng = np.random.default_rng(seed)
    q = bf16_round(rng.standard_normal((nq, Hq, D)).astype(np.float32) * 2)
    k = bf16_round(rng.standard_normal((L, Hkv, D)).astype(np.float32) * 2)
    v = bf16_round(rng.standard_normal((L, Hkv, D)).astype(np.float32) * v_std)
    return q, k, v


def dq(x, s):
    return e4m3_decode(quantize_e4m3(x, s))


def rel_table(Hq, E, seed):
    """A bf16-exact learned relative-bias table [Hq, E]."""
    rng = np.random.default_rng(seed)
    return bf16_round(rng.standard_normal((Hq, E)).astype(np.float32) * 2)


@pytest.mark.parametrize("window,bias", [(0, None), (0, "slopes"), (5, "slopes"), (1, None),
                                         (0, "rel"), (5, "rel")])
def test_bruteforce_matches_vectorised(window, bias):
    q, k, v = tiny()
    L = k.shape[0]
    qs, ks, vs, sm = 0.5, 0.25, 1.5, 0.3
    pos = np.array([L - 3, L - 2, L - 1])
    slopes = geometric_slopes(4) if bias == "slopes" else None
    rel = rel_table(4, 7, 3) if bias == "rel" else None    # extent 7 < distances up to 18
    got = attend_sequence(quantize_q(q, qs), pos, dq(k, ks), dq(v, vs), sm * qs * ks, vs,
                          window, slopes, rel=rel)
    # brute force on explicitly dequantised values (scales applied per element)
    bq = (dq(q, qs) * qs).tolist()
    bk = (dq(k, ks) * ks).tolist()
    bv = (dq(v, vs) * vs).tolist()
    want = np.array(brute_force(bq, pos, bk, bv, sm, window, slopes,
                                None if rel is None else rel.tolist()))
    assert np.max(np.abs(got - want)) < 1e-12 * max(1.0, np.max(np.abs(want)))


def test_fold_equals_explicit_dequant_and_v_linearity():
    q, k, v = tiny(seed=1, L=40)
    L = k.shape[0]
    qs, ks, vs, sm = 0.7, 1.3, 2.5, 1 / math.sqrt(8)
    pos = np.array([L - 1])
    folded = attend_sequence(quantize_q(q[:1], qs), pos, dq(k, ks), dq(v, vs), sm * qs * ks,
                             vs, 0, None)
    explicit = attend_sequence(quantize_q(q[:1], qs) * qs, pos, dq(k, ks) * ks, dq(v, vs) * vs,
                               sm, 1.0, 0, None)
    assert np.max(np.abs(folded - explicit)) <= 1e-12 * np.max(np.abs(explicit))


@pytest.mark.parametrize("chunk", [1, 2, 7, 64])
def test_split_invariance(chunk):
    q, k, v = tiny(seed=2, L=50, nq=4)
    L = k.shape[0]
    pos = np.array([10, 30, 48, 49])
    slopes = geometric_slopes(4)
    args = (quantize_q(q, 1.0), pos, dq(k, 1.0), dq(v, 1.0), 0.35, 2.0, 0, slopes)
    a = attend_sequence(*args)
    b = attend_split(*args, chunk=chunk)
    assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(a)))
    aw = attend_sequence(*args[:6], 9, slopes)
    bw = attend_split(*args[:6], 9, slopes, chunk=chunk)
    assert np.max(np.abs(aw - bw)) < 1e-12 * max(1.0, np.max(np.abs(aw)))


def test_window_reduction():
    q, k, v = tiny(seed=3, L=60, nq=1)
    L, W = 60, 16
    qv = quantize_q(q, 1.0)
    kd, vd = dq(k, 1.0), dq(v, 1.0)
    win = attend_sequence(qv, np.array([L - 1]), kd, vd, 0.4, 1.0, W, None)
    last = attend_sequence(qv, np.array([W - 1]), kd[L - W:], vd[L - W:], 0.4, 1.0, 0, None)
    assert np.max(np.abs(win - last)) < 1e-13
    short = attend_sequence(qv, np.array([9]), kd[:10], vd[:10], 0.4, 1.0, W, None)
    full = attend_sequence(qv, np.array([9]), kd[:10], vd[:10], 0.4, 1.0, 0, None)
    assert np.array_equal(short, full)


def test_zero_query_gives_mean_and_single_key():
    q, k, v = tiny(seed=4, L=23, nq=1)
    vd = dq(v, 1.0)
    out = attend_sequence(np.zeros_like(quantize_q(q, 1.0)), np.array([22]), dq(k, 1.0), vd,
                          0.5, 1.0, 0, None)
    Hq, grp = 4, 2
    for h in range(Hq):
        assert np.max(np.abs(out[0, h] - vd[:, h // grp, :].mean(axis=0))) < 1e-13
    one = attend_sequence(quantize_q(q, 1.0), np.array([22]), dq(k, 1.0), vd, 0.5, 3.0, 1, None)
    for h in range(Hq):
        assert np.max(np.abs(one[0, h] - 3.0 * vd[22, h // grp, :])) < 1e-13


def test_zero_slope_equals_no_bias_and_bias_sign():
    q, k, v = tiny(seed=5, L=30)
    args = (quantize_q(q, 1.0), np.array([27, 28, 29]), dq(k, 1.0), dq(v, 1.0), 0.3, 1.0, 0)
    a = attend_sequence(*args, None)
    b = attend_sequence(*args, np.zeros(4, np.float32))
    assert np.array_equal(a, b)
    bias = relative_bias(0.5, np.array([10]), np.arange(11))
    assert bias[0, 10] == 0.0 and bias[0, 0] == -5.0 and np.all(np.diff(bias[0]) >= 0)
    # the bias is bf16-exact: slope 0.3 at distance 7 rounds to bf16
    b7 = relative_bias(0.3, np.array([7]), np.array([0]))[0, 0]
    assert b7 == float(bf16_round(np.float32(0.3) * np.float32(-7)))
    assert b7 != float(np.float32(0.3) * np.float32(-7))


def test_learned_bias_closed_form_softmax():
    """Q = 0: the scores are the bias alone, so with one-hot V rows the output
    is the softmax of the table entries the keys select. Key j of a query at
    position p reads entry min(p - j, E - 1): the current token the first
    entry, every distance from E - 1 on the last one; heads read their own
    rows; a window keeps only the nearest keys."""
    L, E, Hq, D = 10, 4, 2, 16
    T = np.array([[0.5, -1.25, 2.0, 0.75], [-3.0, 0.0, 1.5, -0.5]], np.float32)
    rng = np.random.default_rng(11)
    k = rng.standard_normal((L, 1, D))
    v = np.zeros((L, 1, D))
    v[np.arange(L), 0, np.arange(L)] = 1.0
    q = np.zeros((1, Hq, D))
    for window, keys in ((0, range(L)), (3, range(L - 3, L))):
        got = attend_sequence(q, np.array([L - 1]), k, v, 0.7, 1.0, window, None, rel=T)[0]
        for h in range(Hq):
            e = {j: float(T[h][min(L - 1 - j, E - 1)]) for j in keys}
            z = sum(math.exp(x) for x in e.values())
            want = np.zeros(D)
            for j, x in e.items():
                want[j] = math.exp(x) / z
            assert np.max(np.abs(got[h] - want)) < 1e-15
    # the lookup itself: distance 0 -> entry 0, distances >= E - 1 -> entry E - 1
    bias = learned_bias(T[0], np.array([9]), np.arange(10))
    assert list(bias[0]) == [0.75] * 7 + [2.0, -1.25, 0.5]


def test_learned_table_of_slope_bias_equals_slope_path():
    """A table holding the slope bias bf16(slope * -d) for every distance
    reproduces the slope path exactly; a shorter table (clamped distances)
    does not."""
    q, k, v = tiny(seed=7, L=40)
    slopes = geometric_slopes(4)
    args = (quantize_q(q, 1.0), np.array([37, 38, 39]), dq(k, 1.0), dq(v, 1.0), 0.3, 1.0, 0)
    a = attend_sequence(*args, slopes)
    for E, same in ((40, True), (64, True), (8, False)):
        T = np.stack([relative_bias(float(sl), np.arange(E), np.zeros(1, np.int64))[:, 0] for sl in slopes])
        b = attend_sequence(*args, None, rel=T)
        assert np.array_equal(a, b) == same


def test_gqa_equals_repeated_kv_heads():
    q, k, v = tiny(seed=6, L=33, Hq=8, Hkv=2)
    pos = np.array([30, 31, 32])
    slopes = geometric_slopes(8)
    g = attend_sequence(quantize_q(q, 1.0), pos, dq(k, 1.0), dq(v, 1.0), 0.3, 1.0, 0, slopes)
    kr = np.repeat(dq(k, 1.0), 4, axis=1)
    vr = np.repeat(dq(v, 1.0), 4, axis=1)
    m = attend_sequence(quantize_q(q, 1.0), pos, kr, vr, 0.3, 1.0, 0, slopes)
    assert np.max(np.abs(g - m)) < 1e-14


def test_paged_wrappers_match_bruteforce_positions():
    """Decode attends at position L-1; prefill's new rows sit at L-Lq+i.
    Checked through the page gather against brute force on the raw tokens."""
    c = make_attn_case("w", 12, [21, 3, 40], [1, 1, 1], 4, 2, 8, slopes=geometric_slopes(4))
    kc, vc = new_cache(c.num_pages, 2, 16, 8)
    k, v = c.k.float().numpy(), c.v.float().numpy()
    store_e4m3(kc, vc, k, v, c.slot_mapping, 0.5, 2.0)
    q = c.q.float().numpy()
    out = paged_decode(q, kc, vc, c.block_table, c.seq_lens, 0.3, 0.25, 0.5, 2.0, 0, c.slopes)
    start = 0
    for b, L in enumerate(c.seq_lens):
        L = int(L)
        kd = (dq(k[start:start + L], 0.5) * 0.5).tolist()
        vd = (dq(v[start:start + L], 2.0) * 2.0).tolist()
        qd = (dq(q[b:b + 1], 0.25) * 0.25).tolist()
        want = np.array(brute_force(qd, [L - 1], kd, vd, 0.3, 0, c.slopes))[0]
        assert np.max(np.abs(out[b] - want)) < 1e-12 * max(1, np.max(np.abs(want)))
        start += L
    # prefill: 2 sequences with 5 and 3 new rows
    c2 = make_attn_case("p", 13, [24, 9], [5, 3], 4, 1, 8, slopes=geometric_slopes(4), window=6)
    kc2, vc2 = new_cache(c2.num_pages, 1, 16, 8)
    k2, v2 = c2.k.float().numpy(), c2.v.float().numpy()
    store_e4m3(kc2, vc2, k2, v2, c2.slot_mapping, 1.0, 1.0)
    q2 = c2.q.float().numpy()
    outp = paged_prefill(q2, c2.cu_q_lens, kc2, vc2, c2.block_table, c2.seq_lens, 0.3, 1.0,
                         1.0, 1.0, 6, c2.slopes)
    start = 0
    for b in range(2):
        L, lq = int(c2.seq_lens[b]), int(c2.q_lens[b])
        r0 = int(c2.cu_q_lens[b])
        kd = dq(k2[start:start + L], 1.0).tolist()
        vd = dq(v2[start:start + L], 1.0).tolist()
        qd = dq(q2[r0:r0 + lq], 1.0).tolist()
        want = np.array(brute_force(qd, list(range(L - lq, L)), kd, vd, 0.3, 6, c2.slopes))
        assert np.max(np.abs(outp[r0:r0 + lq] - want)) < 1e-12 * max(1, np.max(np.abs(want)))
        start += L


def test_zero_length_sequence_outputs_zero():
    c = make_attn_case("z", 14, [0, 17], [1, 1], 4, 2, 8)
    kc, vc = new_cache(c.num_pages, 2, 16, 8)
    store_e4m3(kc, vc, c.k.float().numpy(), c.v.float().numpy(), c.slot_mapping, 1, 1)
    out = paged_decode(c.q.float().numpy(), kc, vc, c.block_table, c.seq_lens, 0.3, 1, 1, 1)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out[1])) and np.any(out[1] != 0)
