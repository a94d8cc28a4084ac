"""GPU parity of the NVFP4 368-byte record store (bit-exact) and of the MLA
decode over those records (within tolerance) against the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_paged_amd as kvq
from oracle.codecs import bf16_round
from oracle.nvfp4 import new_pool, store_records, mla_decode
from workloads import bf16, make_mla_case, config_nvfp4_mla
from workloads.gen import mla_layer_stds
from parity import check_attention

pytestmark = pytest.mark.gpu


def special_tokens():
    """Edge tokens: all zero, an exact two-level grid token (amax 168), a
    token whose e2m1 inputs sit exactly on the rounding midpoints and one bf16
    step either side of them, a token with an all-zero group, tiny
    magnitudes, huge magnitudes."""
    rng = np.random.default_rng(17)
    toks = []
    toks.append(np.zeros(576, np.float32))
    t = np.zeros(576, np.float32)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    t[0:16] = np.tile(grid, 2) * 28.0
    t[0] = 168.0
    t[16:32] = np.tile(grid, 2) * 0.125
    t[512:] = rng.standard_normal(64).astype(np.float32)
    toks.append(t)
    # amax 2688 makes the outer scale 1; groups 1 and 2 have amax 48, so their
    # scale is 8 and x / 8 is exact: group 1 lands on every midpoint of the
    # e2m1 grid (ties go to the even code) and rounds -0.5 / 8 to a signed
    # zero; group 2 sits one bf16 step either side of midpoints and of 6
    t = np.zeros(576, np.float32)
    t[0] = 2688.0
    t[16:32] = [2, -2, 6, -6, 10, -10, 14, -14, 20, -20, 28, -28, 40, -40, 48, -0.5]
    t[32:48] = [19.875, 20.125, -19.875, -20.125, 1.9921875, 2.015625, 39.75, 40.25,
                27.875, 28.125, 48, -48, 5.96875, 6.03125, 13.9375, 14.0625]
    t[512:] = rng.standard_normal(64).astype(np.float32)
    toks.append(t)
    t = rng.standard_normal(576).astype(np.float32)
    t[32:48] = 0.0
    toks.append(t)
    toks.append(rng.standard_normal(576).astype(np.float32) * 1e-30)
    toks.append(rng.standard_normal(576).astype(np.float32) * 1e30)
    t = rng.standard_normal(576).astype(np.float32)
    t[5] = -1000.0       # one dominant element: most group scales tiny
    toks.append(t)
    return bf16_round(np.stack(toks))


@pytest.mark.parametrize("rope_scale", [1.0, 0.37])
def test_store_records_bit_exact(rope_scale):
    rng = np.random.default_rng(3)
    parts = [special_tokens()]
    for std in mla_layer_stds() + [1e-3, 30.0]:
        parts.append(bf16_round((rng.standard_normal((40, 576)) * std).astype(np.float32)))
    x = np.concatenate(parts)
    T = x.shape[0]
    num_pages = (T + 15) // 16 + 3
    slot = rng.permutation(num_pages * 16)[:T].astype(np.int64)
    slot[::7] = -1
    cache = kvq.Nvfp4Cache(num_pages)
    kvq.store(cache, bf16(x).cuda(), None, torch.from_numpy(slot).cuda(), rope_scale)
    torch.cuda.synchronize()
    pool = new_pool(num_pages)
    store_records(pool, x, slot, rope_scale)
    got = cache.records.cpu().numpy()
    bad = np.argwhere(got != pool)
    assert bad.size == 0, bad[:10]


def test_store_full_size_sampled():
    """All 524,288 tokens of the layer with std 0.05; four sequences compared."""
    c = config_nvfp4_mla(layer=0)
    cache = kvq.Nvfp4Cache(c.num_pages)
    kv = c.kv.cuda()
    kvq.store(cache, kv, None, torch.from_numpy(c.slot_mapping).cuda(), c.rope_scale)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(c.seq_lens)])
    tok = np.concatenate([np.arange(starts[b], starts[b + 1]) for b in (0, 9, 20, 31)])
    pool = new_pool(c.num_pages)
    store_records(pool, c.kv.float().numpy()[tok], c.slot_mapping[tok], c.rope_scale)
    pages = np.unique(c.slot_mapping[tok] // 16)
    got = cache.records[torch.from_numpy(pages).cuda()].cpu().numpy()
    assert np.array_equal(got, pool[pages])


def run_mla(c, seqs=None, **kw):
    cache = kvq.Nvfp4Cache(c.num_pages)
    kvq.store(cache, c.kv.cuda(), None, torch.from_numpy(c.slot_mapping).cuda(), c.rope_scale)
    out = kvq.decode(cache, c.q.cuda(), torch.from_numpy(c.block_table).cuda(),
                     torch.from_numpy(c.seq_lens).cuda(), c.max_seq_len, c.softmax_scale,
                     k_scale=c.rope_scale, **kw)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(c.seq_lens)])
    sel = range(c.batch) if seqs is None else seqs
    tok = np.concatenate([np.arange(starts[b], starts[b + 1]) for b in sel])
    pool = new_pool(c.num_pages)
    store_records(pool, c.kv.float().numpy()[tok], c.slot_mapping[tok], c.rope_scale)
    ref = mla_decode(c.q.float().numpy(), pool, c.block_table, c.seq_lens, c.softmax_scale,
                     c.rope_scale, seqs=seqs)
    if seqs is not None:
        return out[torch.tensor(seqs)], ref[seqs]
    return out, ref


@pytest.mark.parametrize("std", [0.05, 1.0, 4.0])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mla_decode_shapes(std, splits):
    c = make_mla_case("mla", 50 + int(std * 10), [1, 15, 16, 17, 300, 1000], layer_std=std,
                      rope_scale=0.8)
    out, ref = run_mla(c, num_splits=splits)
    print(check_attention(out, ref, "mla std %g splits %d" % (std, splits)))


@pytest.mark.parametrize("splits", [8, 12, 40])
def test_mla_decode_many_splits(splits):
    """Split counts at and past the MLA combine's register-prefetch width (8);
    the 17-key sequence leaves most splits without a key."""
    c = make_mla_case("mla_splits", 70 + splits, [3000, 1500, 17], layer_std=1.0, rope_scale=1.0)
    out, ref = run_mla(c, num_splits=splits)
    check_attention(out, ref, "mla splits %d" % splits)


def test_mla_decode_zero_length_and_poison():
    c = make_mla_case("mla0", 61, [0, 33, 5], layer_std=1.0, spare_frac=2.0)
    out, ref = run_mla(c)
    assert torch.all(out[0] == 0)
    assert torch.all(torch.isfinite(out.float()))
    check_attention(out, ref, "mla zero/poison")


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_mla_decode_full_size_sampled(layer):
    """Batch 32 x 16,384 tokens, each of the four layer stds (0.05, 4 and two
    uniform draws); four sequences compared with the oracle."""
    c = config_nvfp4_mla(layer=layer)
    out, ref = run_mla(c, seqs=[0, 7, 19, 31])
    print(check_attention(out, ref, "nvfp4 mla layer %d" % layer))


def run_mla_prefill(c, q_lens, seed, rows=None):
    """NVFP4 prefill: the case's records hold every token; q_lens new query
    rows per sequence (the last tokens) are drawn here."""
    from oracle.nvfp4 import mla_prefill
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = bf16(rng.standard_normal((int(cu[-1]), 16, 576)).astype(np.float32))
    cache = kvq.Nvfp4Cache(c.num_pages)
    kvq.store(cache, c.kv.cuda(), None, torch.from_numpy(c.slot_mapping).cuda(), c.rope_scale)
    out = kvq.prefill(cache, q.cuda(), torch.from_numpy(cu).cuda(), int(q_lens.max()),
                      torch.from_numpy(c.block_table).cuda(), torch.from_numpy(c.seq_lens).cuda(),
                      c.max_seq_len, c.softmax_scale, k_scale=c.rope_scale)
    torch.cuda.synchronize()
    pool = new_pool(c.num_pages)
    store_records(pool, c.kv.float().numpy(), c.slot_mapping, c.rope_scale)
    ref = mla_prefill(q.float().numpy(), cu, pool, c.block_table, c.seq_lens, c.softmax_scale,
                      c.rope_scale, rows=rows)
    if rows is not None:
        return out[torch.tensor(rows)], ref[rows]
    return out, ref


@pytest.mark.parametrize("std", [0.05, 1.0, 4.0])
def test_mla_prefill_shapes(std):
    """Ragged new-token counts, a whole-sequence prefill, a sequence without
    new tokens, partial last pages."""
    c = make_mla_case("mla_pf", 70 + int(std * 10), [40, 17, 300, 9, 1000], layer_std=std, rope_scale=0.8)
    out, ref = run_mla_prefill(c, [5, 17, 1, 0, 129], 71)
    print(check_attention(out, ref, "mla prefill std %g" % std))


def test_mla_prefill_long_sampled():
    """Two sequences of 8,192 keys with 256 and 64 new tokens; 40 sampled rows."""
    c = make_mla_case("mla_pf_long", 72, [8192, 8192], layer_std=1.0)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 255, 256, 319] + list(rng.choice(320, 36, replace=False))))
    out, ref = run_mla_prefill(c, [256, 64], 73, rows=rows)
    print(check_attention(out, ref, "mla prefill 2 x 8192"))


def test_mla_prefill_one_token_equals_decode():
    """One new token per sequence is decode: the prefill rows match the
    single-split decode output (same per-key arithmetic; the prefill kernel
    sums each 576-dim dot product in one pass, the decode in two 256-dim
    halves plus RoPE, so the bits may differ by rounding) and the oracle."""
    c = make_mla_case("mla_pf1", 74, [1, 16, 17, 300, 2049], layer_std=1.0)
    cache = kvq.Nvfp4Cache(c.num_pages)
    kvq.store(cache, c.kv.cuda(), None, torch.from_numpy(c.slot_mapping).cuda(), c.rope_scale)
    bt = torch.from_numpy(c.block_table).cuda()
    sl = torch.from_numpy(c.seq_lens).cuda()
    q = c.q.cuda()
    dec = kvq.decode(cache, q, bt, sl, c.max_seq_len, c.softmax_scale, num_splits=1)
    cu = torch.arange(c.batch + 1, dtype=torch.int32, device="cuda")
    pf = kvq.prefill(cache, q, cu, 1, bt, sl, c.max_seq_len, c.softmax_scale)
    torch.cuda.synchronize()
    d, f = dec.float(), pf.float()
    assert float((f - d).norm() / d.norm()) < 1e-3
    assert bool(((f - d).abs() <= 2e-2 * d.abs().clamp(min=1.0)).all())
    pool = new_pool(c.num_pages)
    store_records(pool, c.kv.float().numpy(), c.slot_mapping, c.rope_scale)
    ref = mla_decode(c.q.float().numpy(), pool, c.block_table, c.seq_lens, c.softmax_scale, c.rope_scale)
    check_attention(pf, ref, "mla prefill, one new token")


def test_mla_prefill_full_size_sampled():
    """The prefill workload the bench times (4 x 16,384 tokens, last 1,024
    new), in the same launch; 24 sampled rows against the oracle."""
    from oracle.nvfp4 import mla_prefill
    from workloads import config_nvfp4_mla_prefill
    c = config_nvfp4_mla_prefill()
    cache = kvq.Nvfp4Cache(c.num_pages)
    kvq.store(cache, c.kv.cuda(), None, torch.from_numpy(c.slot_mapping).cuda(), c.rope_scale)
    cu = c.cu_q_lens
    out = kvq.prefill(cache, c.q.cuda(), torch.from_numpy(cu).cuda(), int(c.q_lens.max()),
                      torch.from_numpy(c.block_table).cuda(), torch.from_numpy(c.seq_lens).cuda(),
                      c.max_seq_len, c.softmax_scale, k_scale=c.rope_scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = sorted(set([0, 1023, 1024, int(cu[-1]) - 1] + list(rng.choice(int(cu[-1]), 20, replace=False))))
    pool = new_pool(c.num_pages)
    store_records(pool, c.kv.float().numpy(), c.slot_mapping, c.rope_scale)
    ref = mla_prefill(c.q.float().numpy(), cu, pool, c.block_table, c.seq_lens, c.softmax_scale,
                      c.rope_scale, rows=rows)
    print(check_attention(out[torch.tensor(rows)], ref[rows], "nvfp4 mla prefill full size"))


@pytest.mark.parametrize("outer", [1.0, 0.0137, 2.0 ** -10])
def test_store_static_outer_scale_bit_exact(outer):
    """The static outer-scale store against the oracle's static records, over
    the edge tokens and magnitudes from 1e-3 to 30 (subnormal and flushed
    group scales at the small end, saturated ones at the large end)."""
    rng = np.random.default_rng(21)
    parts = [special_tokens()]
    for std in (30.0, 1.0, 0.05, 0.01, 0.002, 1e-3):
        parts.append(bf16_round((rng.standard_normal((24, 576)) * std).astype(np.float32)))
    x = np.concatenate(parts)
    T = x.shape[0]
    num_pages = (T + 15) // 16 + 2
    slot = rng.permutation(num_pages * 16)[:T].astype(np.int64)
    slot[::9] = -1
    cache = kvq.Nvfp4Cache(num_pages)
    kvq.store_nvfp4_static(cache, bf16(x).cuda(), torch.from_numpy(slot).cuda(), 0.5, outer)
    torch.cuda.synchronize()
    pool = new_pool(num_pages)
    store_records(pool, x, slot, 0.5, static_s2=outer)
    got = cache.records.cpu().numpy()
    bad = np.argwhere(got != pool)
    assert bad.size == 0, bad[:10]


def e2m1_input_tokens(seed: int):
    """Every bf16 value of magnitude 2^-10 up to 48, both signs, spread in a
    seeded random order over groups whose first element is +-48. Element 0 of
    each token is 2688, so the outer scale is exactly 1; every other group has
    amax 48, so its scale is 8 (exact in e4m3) and x / 8 is exact: the e2m1
    inputs are every bf16-representable value of magnitude up to 6, each
    rounding midpoint and its neighbours among them."""
    mags = []
    for e in range(-10, 6):
        m = (1.0 + np.arange(128) / 128.0) * 2.0 ** e
        mags.append(m[m <= 48.0])
    mags = np.concatenate(mags).astype(np.float32)
    vals = np.concatenate([mags, -mags])
    rng = np.random.default_rng(seed)
    vals = vals[rng.permutation(vals.size)]
    per_token = 31 * 15                       # groups 1..31, 15 free slots each
    T = (vals.size + per_token - 1) // per_token
    x = np.zeros((T, 576), np.float32)
    x[:, 0] = 2688.0
    lat = x[:, 16:512].reshape(T, 31, 16)
    lat[:, :, 0] = np.where(rng.random((T, 31)) < 0.5, 48.0, -48.0)
    free = np.zeros(T * per_token, np.float32)
    free[:vals.size] = vals
    lat[:, :, 1:] = free.reshape(T, 31, 15)
    x[:, 16:512] = lat.reshape(T, 496)
    x[:, 512:] = x[:, 16:80]
    return x


@pytest.mark.parametrize("outer", [None, 1.0, 2.0 ** -20])
def test_store_every_e2m1_input_bit_exact(outer):
    """Every bf16 value up to the e2m1 maximum as an e2m1 input through the
    NVFP4 store, bit-exact against the oracle: with the per-token outer scale,
    with a static one of 1 (the same inputs), and with a tiny static one that
    saturates the group scales at 448 and sends the inputs far past 6 (clip)."""
    x = e2m1_input_tokens(9)
    assert np.array_equal(bf16_round(x), x)
    T = x.shape[0]
    num_pages = (T + 15) // 16 + 1
    slot = np.random.default_rng(6).permutation(num_pages * 16)[:T].astype(np.int64)
    cache = kvq.Nvfp4Cache(num_pages)
    xs, ss = bf16(x).cuda(), torch.from_numpy(slot).cuda()
    if outer is None:
        kvq.store(cache, xs, None, ss, 1.0)
    else:
        kvq.store_nvfp4_static(cache, xs, ss, 1.0, outer)
    torch.cuda.synchronize()
    pool = new_pool(num_pages)
    if outer is None:
        store_records(pool, x, slot, 1.0)
    else:
        store_records(pool, x, slot, 1.0, static_s2=outer)
    got = cache.records.cpu().numpy()
    bad = np.argwhere(got != pool)
    assert bad.size == 0, bad[:10]


def test_static_outer_scale_ab_through_decode():
    """A/B of the outer scale through the GPU store and MLA decode: relative
    L2 error of the decode output against attention over the unquantized
    tokens. The per-token scale stays near 0.095 at every magnitude; a static
    scale of 1.0 degrades as the latents shrink and collapses once group
    scales flush to zero."""
    from oracle.nvfp4 import mla_exact
    errs = {}
    for std in (1.0, 0.02, 0.01, 0.002):
        c = make_mla_case("ab", 90, [1024] * 4, layer_std=std)
        exact = mla_exact(c.q.float().numpy(), c.kv.float().numpy(), c.seq_lens, c.softmax_scale)
        slot = torch.from_numpy(c.slot_mapping).cuda()
        row = []
        for static in (False, True):
            cache = kvq.Nvfp4Cache(c.num_pages)
            if static:
                kvq.store_nvfp4_static(cache, c.kv.cuda(), slot, 1.0, 1.0)
            else:
                kvq.store(cache, c.kv.cuda(), None, slot, 1.0)
            out = kvq.decode(cache, c.q.cuda(), torch.from_numpy(c.block_table).cuda(),
                             torch.from_numpy(c.seq_lens).cuda(), c.max_seq_len, c.softmax_scale)
            o = out.float().cpu().numpy().astype(np.float64)
            row.append(float(np.linalg.norm(o - exact) / np.linalg.norm(exact)))
        errs[std] = row
    print(errs)
    for std, (dyn, sta) in errs.items():
        assert 0.085 < dyn < 0.11, (std, dyn)
    assert abs(errs[1.0][1] - errs[1.0][0]) < 5e-3
    assert errs[0.01][1] > 1.25 * errs[0.01][0]
    assert errs[0.002][1] > 0.5
    assert errs[1.0][1] < errs[0.02][1] + 5e-3 < errs[0.01][1] + 5e-3 < errs[0.002][1]
