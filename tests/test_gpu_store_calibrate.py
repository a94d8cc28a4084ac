"""GPU parity of quant-on-store and amax calibration: stored bytes and scales
must be bit-identical to the oracle's."""
import numpy as np
import pytest
import torch

import fp4_quantized_paged_amd as kvq
from oracle.codecs import bf16_bits_to_f32
from oracle.kvcache import new_cache, store_e4m3, calibrate_amax, quantize_e4m3
from oracle.calibration import band_counts, scale_from_amax
from workloads import bf16, config_tiny_decode, config_batched_decode, make_attn_case
from parity import DeviceCase, oracle_scales, oracle_cache, seq_tokens

pytestmark = pytest.mark.gpu


def all_patterns(hkv, d):
    """Every bf16 bit pattern, as [T, hkv, d] tokens (T*hkv*d = 65536)."""
    bits = np.arange(65536, dtype=np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return x.reshape(-1, hkv, d)


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.5, 3.0), (20.0 / 448, 1272.0 / 448)])
@pytest.mark.parametrize("layout", ["pages", "scattered"])
def test_store_all_bf16_patterns(scales, layout):
    hkv, d = 4, 128
    k = all_patterns(hkv, d)                     # 128 tokens
    v = torch.flip(k, dims=[0]).contiguous()
    T = k.shape[0]
    num_pages = 2 * T // 16 + 4
    if layout == "pages":
        slot = np.arange(T, dtype=np.int64) + 32          # whole pages, in order
    else:
        rng = np.random.default_rng(1)
        slot = rng.permutation(num_pages * 16)[:T].astype(np.int64)
    cache = kvq.E4M3Cache(num_pages, hkv, d)
    kvq.store(cache, k.cuda(), v.cuda(), torch.from_numpy(slot).cuda(), *scales)
    torch.cuda.synchronize()
    kc, vc = new_cache(num_pages, hkv, 16, d)
    store_e4m3(kc, vc, k.float().numpy(), v.float().numpy(), slot, *scales)
    gk, gv = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    nan_k = np.isnan(k.float().numpy())
    # NaN inputs must give a NaN code (either sign); every other byte exact
    ok_k = (gk == kc)
    if nan_k.any():
        pages = slot // 16
        for t, h, dd in zip(*np.nonzero(nan_k)):
            b = gk[pages[t], h, slot[t] % 16, dd]
            assert b & 0x7F == 0x7F
            ok_k[pages[t], h, slot[t] % 16, dd] = True
    assert ok_k.all(), np.argwhere(~ok_k)[:5]
    nan_v = np.isnan(v.float().numpy())
    ok_v = (gv == vc)
    pages = slot // 16
    for t, h, dd in zip(*np.nonzero(nan_v)):
        assert gv[pages[t], h, dd, slot[t] % 16] & 0x7F == 0x7F
        ok_v[pages[t], h, dd, slot[t] % 16] = True
    assert ok_v.all(), np.argwhere(~ok_v)[:5]


@pytest.mark.parametrize("hkv", [16, 32])
def test_store_wide_rows(hkv):
    """Whole pages in order with 16 and 32 KV heads of 128 dims: the largest
    row whose two V page images fit the staged path, and one that takes the
    in-place path."""
    d, T = 128, 96
    rng = np.random.default_rng(hkv)
    k = bf16(rng.standard_normal((T, hkv, d)).astype(np.float32) * 3.0)
    v = bf16(rng.standard_normal((T, hkv, d)).astype(np.float32) * 8.0)
    num_pages = T // 16 + 3
    slot = np.arange(T, dtype=np.int64) + 32
    cache = kvq.E4M3Cache(num_pages, hkv, d)
    kvq.store(cache, k.cuda(), v.cuda(), torch.from_numpy(slot).cuda(), 0.05, 0.1)
    torch.cuda.synchronize()
    kc, vc = new_cache(num_pages, hkv, 16, d)
    store_e4m3(kc, vc, k.float().numpy(), v.float().numpy(), slot, 0.05, 0.1)
    assert np.array_equal(cache.k.cpu().numpy(), kc)
    assert np.array_equal(cache.v.cpu().numpy(), vc)


def test_store_tiny_decode_config_bytes():
    c = config_tiny_decode()
    dc = DeviceCase(c)
    s = dc.calibrate()
    dc.store_all(s)
    torch.cuda.synchronize()
    kc, vc = oracle_cache(c, oracle_scales(c))
    assert np.array_equal(dc.cache.k.cpu().numpy(), kc)
    assert np.array_equal(dc.cache.v.cpu().numpy(), vc)


def test_store_negative_slots_and_zero_tokens():
    c = make_attn_case("neg", 21, [40, 33], [1, 1], 4, 2, 64)
    dc = DeviceCase(c)
    slot = c.slot_mapping.copy()
    slot[::5] = -1
    kvq.store(dc.cache, dc.k, dc.v, torch.from_numpy(slot).cuda(), 0.75, 1.5)
    kvq.store(dc.cache, dc.k[:0], dc.v[:0], dc.slot[:0], 0.75, 1.5)  # no-op
    torch.cuda.synchronize()
    kc, vc = new_cache(c.num_pages, 2, 16, 64)
    store_e4m3(kc, vc, c.k.float().numpy(), c.v.float().numpy(), slot, 0.75, 1.5)
    assert np.array_equal(dc.cache.k.cpu().numpy(), kc)
    assert np.array_equal(dc.cache.v.cpu().numpy(), vc)


@pytest.fixture(scope="module")
def batched():
    c = config_batched_decode()
    return c, DeviceCase(c)


def test_calibrate_batched_decode_bit_exact(batched):
    c, dc = batched
    for name, x in (("k", c.k), ("v", c.v), ("q", c.q)):
        amax_g, scale_g = kvq.calibrate_amax(getattr(dc, name))
        amax_o, scale_o = calibrate_amax(x.float().numpy())
        assert amax_g.item() == float(amax_o), name
        assert np.float32(scale_g.item()) == scale_o, name
    # Q and K were generated with amax 20
    assert kvq.calibrate_amax(dc.k)[0].item() == 20.0


def test_calibrate_running_slots_and_empty(batched):
    c, dc = batched
    x = dc.v[:100000]
    amax = torch.zeros(1, device="cuda")
    for c0 in range(0, 100000, 30001):
        kvq.calibrate_amax(x[c0:c0 + 30001], amax=amax)
    one = kvq.calibrate_amax(x)[0]
    assert amax.item() == one.item()
    # skipped rows: drop the row holding the maximum
    xv = c.v[:100000].float().numpy().reshape(100000, -1)
    big = int(np.argmax(np.abs(xv).max(axis=1)))
    slot = np.arange(100000, dtype=np.int64)
    slot[big] = -1
    a_g, s_g = kvq.calibrate_amax(x, torch.from_numpy(slot).cuda())
    a_o, s_o = calibrate_amax(xv, slot)
    assert a_g.item() == float(a_o) and np.float32(s_g.item()) == s_o
    # empty input leaves the running value and still writes the scale
    prev = torch.tensor([3.5], device="cuda")
    a_e, s_e = kvq.calibrate_amax(x[:0], amax=prev)
    assert a_e.item() == 3.5 and np.float32(s_e.item()) == np.float32(3.5) / np.float32(448)


def test_store_batched_decode_sampled(batched):
    """Full-size bulk store (524,288 tokens) with calibrated K and v_scale 3.0;
    three whole sequences compared byte for byte, plus a v_scale 1.0 pass where
    the V outliers saturate."""
    c, dc = batched
    s_gpu = dc.calibrate()
    s_or = oracle_scales(c)
    assert s_gpu == s_or
    dc.store_all(s_gpu)
    torch.cuda.synchronize()
    seqs = [0, 31, 63]
    tok = seq_tokens(c, seqs)
    kc, vc = oracle_cache(c, s_or, tokens=tok)
    pages = np.unique(c.slot_mapping[tok] // 16)
    gk = dc.cache.k[torch.from_numpy(pages).cuda()].cpu().numpy()
    gv = dc.cache.v[torch.from_numpy(pages).cuda()].cpu().numpy()
    assert np.array_equal(gk, kc[pages])
    assert np.array_equal(gv, vc[pages])
    # saturation pass at v_scale 1.0 on the tokens holding outliers
    vv = c.v.float().numpy()
    out_tok = np.unique(np.nonzero(np.abs(vv) >= 448)[0])[:2048]
    cache1 = kvq.E4M3Cache(c.num_pages, 4, 128)
    i = torch.from_numpy(out_tok).cuda()
    kvq.store(cache1, dc.k[i].contiguous(), dc.v[i].contiguous(), dc.slot[i], 1.0, 1.0)
    torch.cuda.synchronize()
    slot = c.slot_mapping[out_tok]
    gv1 = cache1.v.cpu().numpy()[slot // 16, :, :, slot % 16]
    want = quantize_e4m3(vv[out_tok], 1.0)
    assert np.array_equal(gv1, want)
    assert np.sum((want & 0x7F) == 0x7E) > 0


def test_store_deterministic():
    c = make_attn_case("det", 22, [300, 129], [1, 1], 8, 4, 128)
    a, b = DeviceCase(c), DeviceCase(c)
    for dc in (a, b):
        kvq.store(dc.cache, dc.k, dc.v, dc.slot, 0.3, 0.7)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.k, b.cache.k) and torch.equal(a.cache.v, b.cache.v)


@pytest.mark.parametrize("scale", [1.0, 2.0, 3.0, 0.125, 20.0 / 448, 0.7, 1e-3, 1e4, 3.3e-38])
def test_band_counts_all_bf16_patterns(scale):
    """Clip and flush-to-zero counts over every bf16 pattern, bit-exact."""
    x = all_patterns(4, 128).cuda()
    got = kvq.band_counts(x, scale)
    torch.cuda.synchronize()
    want = band_counts(x.float().cpu().numpy(), scale)
    assert tuple(got.cpu().tolist()) == want
    if scale == 1.0:
        assert want == (30528, 29952)


def test_band_counts_slots_and_running_total():
    rng = np.random.default_rng(8)
    x = bf16(rng.standard_normal((300, 4, 64)).astype(np.float32) * 200.0)
    x[::17, 0, :8] = bf16(np.full(8, 1e-5, np.float32))
    slot = np.arange(300, dtype=np.int64)
    slot[::3] = -1
    xd = x.cuda()
    counts = kvq.band_counts(xd, 1.0, torch.from_numpy(slot).cuda())
    counts = kvq.band_counts(xd[:0], 1.0, counts=counts)            # no rows: unchanged
    counts = kvq.band_counts(xd, 0.5, counts=counts)                # running total
    torch.cuda.synchronize()
    xn = x.float().numpy()
    a = band_counts(xn, 1.0, slot)
    b = band_counts(xn, 0.5)
    assert tuple(counts.cpu().tolist()) == (a[0] + b[0], a[1] + b[1])
    assert a[0] > 0 and a[1] > 0


def test_band_counts_batched_decode_v(batched):
    """V of the batched-decode workload (outliers up to 1,272): exact counts on
    three sequences selected by the slot mask; over all 524,288 rows nothing
    clips at scale 3 and the outliers clip at scale 1."""
    c, dc = batched
    seqs = [0, 31, 63]
    tok = seq_tokens(c, seqs)
    mask = np.full(c.v.shape[0], -1, np.int64)
    mask[tok] = 0
    vn = c.v.float().numpy()
    for s in (1.0, 3.0):
        got = kvq.band_counts(dc.v, s, torch.from_numpy(mask).cuda())
        torch.cuda.synchronize()
        assert tuple(got.cpu().tolist()) == band_counts(vn[tok], s)
    full3 = kvq.band_counts(dc.v, 3.0)
    full1 = kvq.band_counts(dc.v, 1.0)
    torch.cuda.synchronize()
    assert full3[0].item() == 0
    assert full1[0].item() == int(np.count_nonzero(np.abs(vn) > 448))


def test_scale_rules_match_oracle():
    rng = np.random.default_rng(9)
    vals = np.concatenate([[0.0, 1e-30, 448.0, 449.0, 1272.0, 812.0, 73.5, 55.8, 344.0, 345.0, 3e38],
                           rng.lognormal(1.0, 4.0, 200)]).astype(np.float32)
    amax = torch.from_numpy(vals).cuda()
    for rule in (kvq.SCALE_AMAX_448, kvq.SCALE_CEIL_BF16, kvq.SCALE_SAFETY_1P3):
        out = torch.empty_like(amax)
        for i in range(len(vals)):
            kvq.scale_from_amax(amax[i:i + 1], rule, out[i:i + 1])
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = np.array([scale_from_amax(a, rule) for a in vals], np.float32)
        bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, (rule, vals[bad[:5]], got[bad[:5]], want[bad[:5]])
