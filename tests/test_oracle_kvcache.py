"""Pins for the oracle's store and calibration: byte placement, slot skipping,
saturation of the V outliers, and closed forms of the amax/448 rule."""
import numpy as np

from oracle.codecs import e4m3_decode, bf16_round, E4M3_TABLE
from oracle.kvcache import (quantize_e4m3, new_cache, store_e4m3, gather_tokens,
                            calibrate_amax)
from workloads import make_attn_case


def small_case():
    return make_attn_case("t", 7, [37, 5, 16], [1, 1, 1], 4, 2, 8, v_std=8.0,
                          v_outlier_frac=0.05)


def test_store_places_every_byte():
    c = small_case()
    kc, vc = new_cache(c.num_pages, c.num_kv_heads, 16, c.head_dim)
    k = c.k.float().numpy()
    v = c.v.float().numpy()
    store_e4m3(kc, vc, k, v, c.slot_mapping, 0.5, 3.0)
    kq = quantize_e4m3(k, 0.5)
    vq = quantize_e4m3(v, 3.0)
    # explicit loops, independent of the vectorised placement
    for t in range(k.shape[0]):
        page, off = divmod(int(c.slot_mapping[t]), 16)
        for h in range(c.num_kv_heads):
            for d in range(c.head_dim):
                assert kc[page, h, off, d] == kq[t, h, d]
                assert vc[page, h, d, off] == vq[t, h, d]
    # pages never assigned keep the poison byte
    used = set((c.slot_mapping // 16).tolist())
    for p in range(c.num_pages):
        if p not in used:
            assert np.all(kc[p] == 0x7F) and np.all(vc[p] == 0x7F)


def test_store_skips_negative_slots_and_gather_inverts():
    c = small_case()
    kc, vc = new_cache(c.num_pages, c.num_kv_heads, 16, c.head_dim)
    slot = c.slot_mapping.copy()
    slot[::3] = -1
    k = c.k.float().numpy()
    v = c.v.float().numpy()
    store_e4m3(kc, vc, k, v, slot, 1.0, 1.0)
    for t in range(k.shape[0]):
        if slot[t] < 0:
            page, off = divmod(int(c.slot_mapping[t]), 16)
            assert np.all(kc[page, :, off, :] == 0x7F)
            assert np.all(vc[page, :, :, off] == 0x7F)
    store_e4m3(kc, vc, k, v, c.slot_mapping, 1.0, 1.0)
    start = 0
    for b, L in enumerate(c.seq_lens):
        gk, gv = gather_tokens(kc, vc, c.block_table[b], int(L))
        assert np.array_equal(gk, quantize_e4m3(k[start:start + L], 1.0))
        assert np.array_equal(gv, quantize_e4m3(v[start:start + L], 1.0))
        start += int(L)


def test_v_outliers_saturate_at_unit_scale_not_at_three():
    # max |V| 1,272: clipped at v_scale 1, exactly representable range at 3
    x = np.array([1272.0, -1272.0, 448.0, 1000.0], dtype=np.float32)
    assert list(quantize_e4m3(x, 1.0)) == [0x7E, 0xFE, 0x7E, 0x7E]
    q3 = quantize_e4m3(x, 3.0)
    assert np.all(np.abs(e4m3_decode(q3)) < 448.0)
    assert abs(e4m3_decode(q3)[0] * 3.0 - 1272.0) / 1272.0 < 2 ** -4


def test_calibrate_closed_forms():
    rng = np.random.default_rng(2)
    x = bf16_round((rng.standard_normal((300, 64)) * 7).astype(np.float32))
    amax, scale = calibrate_amax(x)
    assert amax == np.max(np.abs(x))
    # scale * 448 within one ulp of amax
    assert abs(float(scale) * 448.0 - float(amax)) <= np.spacing(np.float32(amax))
    # the largest element stores as the saturation code
    idx = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    code = quantize_e4m3(x[idx], scale)
    assert code in (0x7E, 0xFE)
    # no element exceeds the e4m3 range after scaling
    q = quantize_e4m3(x, scale)
    assert not np.any((q & 0x7F) == 0x7F)


def test_calibrate_running_and_slots():
    rng = np.random.default_rng(9)
    x = bf16_round(rng.standard_normal((1000, 32)).astype(np.float32))
    one, _ = calibrate_amax(x)
    run = 0.0
    for c0 in range(0, 1000, 137):
        run, _ = calibrate_amax(x[c0:c0 + 137], prev_amax=run)
    assert run == one
    slot = np.arange(1000)
    big = int(np.argmax(np.abs(x).max(axis=1)))
    slot[big] = -1
    a_skip, _ = calibrate_amax(x, slot)
    rows = np.delete(x, big, axis=0)
    assert a_skip == np.max(np.abs(rows)) and a_skip < one
    # empty input leaves the running value
    a_empty, s_empty = calibrate_amax(x[:0], prev_amax=3.5)
    assert a_empty == np.float32(3.5) and s_empty == np.float32(3.5) / np.float32(448)


def test_decoded_table_matches_bitfields_for_all_codes():
    # independent decode via float construction from fields
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(E4M3_TABLE[c])
            continue
        val = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert E4M3_TABLE[c] == (-val if s else val)
