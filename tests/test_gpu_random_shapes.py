"""Seeded random shapes for the e4m3 decode and chunked prefill against the
fp64 oracle: sequence counts and lengths (empty, one page, ragged, tens of
thousands of keys), GQA groups 1-16, head_dim 64/128, windows, slope and
learned-table biases, forced and planned split counts, fp16 and two-term e4m3
P. Each case is drawn from its own seed, so a failure names a reproducible
shape."""
import numpy as np
import pytest
import torch

from oracle.attention import paged_decode, paged_prefill
from workloads import make_attn_case, geometric_slopes
from parity import DeviceCase, oracle_scales, oracle_cache, check_attention

pytestmark = pytest.mark.gpu

HEADS = [(8, 1), (16, 2), (32, 4), (12, 3), (32, 2), (64, 8), (8, 8), (16, 4)]


def _bias(rng, hq):
    kind = ["none", "slope", "table"][int(rng.integers(3))]
    if kind == "slope":
        return kind, {"slopes": geometric_slopes(hq)}
    if kind == "table":
        return kind, {"rel_extent": int(rng.choice([1, 128, 1024, 5000]))}
    return kind, {}


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    rng = np.random.default_rng(9100 + seed)
    B = int(rng.integers(1, 5))
    long = rng.random() < 0.3
    lens = [int(x) for x in rng.integers(20000 if long else 0, 70000 if long else 3000, B)]
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = 128 if rng.random() < 0.7 else 64
    window = int(rng.choice([0, 0, 0, 100, 512, 4096]))
    kind, kw = _bias(rng, hq)
    splits = int(rng.choice([0, 0, 0, 1, 3, 17]))
    c = make_attn_case("rdecode", 9100 + seed, lens, [1] * B, hq, hkv, d, v_std=2.0, window=window, **kw)
    dc = DeviceCase(c)
    s = dc.calibrate()
    so = oracle_scales(c)
    assert s == so
    dc.store_all(s)
    out = dc.decode(s, num_splits=splits)
    torch.cuda.synchronize()
    kc, vc = oracle_cache(c, so)
    ref = paged_decode(c.q.float().numpy(), kc, vc, c.block_table, c.seq_lens, c.softmax_scale,
                       so["q"], so["k"], so["v"], c.window, c.slopes, rel=c.rel)
    print(check_attention(out, ref, "decode %s h%d/%d D%d w%d %s splits %d" % (lens, hq, hkv, d, window, kind, splits)))


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(seed):
    rng = np.random.default_rng(9200 + seed)
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(1, 1500, B)]
    qlens = [int(min(n, rng.integers(0, 600))) for n in lens]
    if sum(qlens) == 0:
        qlens[0] = lens[0]
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    window = int(rng.choice([0, 0, 64, 300]))
    kind, kw = _bias(rng, hq)
    mode = {} if rng.random() < 0.7 else {"fp8_p2": True}
    c = make_attn_case("rprefill", 9200 + seed, lens, qlens, hq, hkv, 128, v_std=2.0, window=window, **kw)
    dc = DeviceCase(c)
    s = dc.calibrate()
    so = oracle_scales(c)
    assert s == so
    dc.store_all(s)
    out = dc.prefill(s, **mode)
    torch.cuda.synchronize()
    kc, vc = oracle_cache(c, so)
    ref = paged_prefill(c.q.float().numpy(), c.cu_q_lens, kc, vc, c.block_table, c.seq_lens, c.softmax_scale,
                        so["q"], so["k"], so["v"], c.window, c.slopes, rel=c.rel)
    print(check_attention(out, ref, "prefill %s q %s h%d/%d w%d %s %s" % (lens, qlens, hq, hkv, window, kind, mode)))


@pytest.mark.parametrize("seed", range(8))
def test_random_nvfp4_decode_and_prefill(seed):
    """NVFP4 records: random batch, lengths (0 to 6,000 keys), layer std and
    RoPE scale, planned or forced splits for the decode, then a prefill of a
    random number of each sequence's last tokens over the same records."""
    from oracle.nvfp4 import new_pool, store_records, mla_decode, mla_prefill
    from workloads import make_mla_case, bf16
    import fp4_quantized_paged_amd as kvq
    rng = np.random.default_rng(9300 + seed)
    B = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 6000, B)]
    std = float(rng.choice([0.05, 0.5, 1.0, 4.0]))
    rope = float(rng.choice([0.5, 1.0, 2.0]))
    splits = int(rng.choice([0, 0, 1, 5, 24]))
    c = make_mla_case("rnv", 9300 + seed, lens, layer_std=std, rope_scale=rope)
    cache = kvq.Nvfp4Cache(c.num_pages)
    kvq.store(cache, c.kv.cuda(), None, torch.from_numpy(c.slot_mapping).cuda(), c.rope_scale)
    bt = torch.from_numpy(c.block_table).cuda()
    sl = torch.from_numpy(c.seq_lens).cuda()
    out = kvq.decode(cache, c.q.cuda(), bt, sl, c.max_seq_len, c.softmax_scale, k_scale=c.rope_scale,
                     num_splits=splits)
    q_lens = np.array([int(rng.integers(0, min(n, 300) + 1)) for n in lens], dtype=np.int32)
    if q_lens.sum() == 0:
        q_lens[int(np.argmax(lens))] = min(max(lens), 1)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    qp = bf16(rng.standard_normal((int(cu[-1]), 16, 576)).astype(np.float32))
    outp = kvq.prefill(cache, qp.cuda(), torch.from_numpy(cu).cuda(), max(int(q_lens.max()), 1), bt, sl,
                       c.max_seq_len, c.softmax_scale, k_scale=c.rope_scale)
    torch.cuda.synchronize()
    pool = new_pool(c.num_pages)
    store_records(pool, c.kv.float().numpy(), c.slot_mapping, c.rope_scale)
    ref = mla_decode(c.q.float().numpy(), pool, c.block_table, c.seq_lens, c.softmax_scale, c.rope_scale)
    print(check_attention(out, ref, "nvfp4 decode %s std %g rope %g splits %d" % (lens, std, rope, splits)))
    if cu[-1] > 0:
        refp = mla_prefill(qp.float().numpy(), cu, pool, c.block_table, c.seq_lens, c.softmax_scale, c.rope_scale)
        print(check_attention(outp, refp, "nvfp4 prefill %s q %s" % (lens, q_lens.tolist())))
