"""GPU parity on the kernel-benchmark shapes of the vLLM PR 54705 evidence
document ("Tier 1: kernel performance"): single-stream decode over 65,536
keys on a TP4 rank's heads, the q = 8,192 sliding-window (local) prefill on
TP1 heads with the learned relative bias, and the write path's quant-on-store
at two head configurations and 33 / 2,048 / 16,384 tokens."""
import numpy as np
import pytest
import torch

import fp4_quantized_paged_amd as kvq
from oracle.attention import paged_decode, paged_prefill
from oracle.kvcache import new_cache, store_e4m3, calibrate_amax
from workloads import config_single_stream_decode, config_local_prefill, write_path_tokens
from parity import DeviceCase, oracle_scales, oracle_cache, check_attention

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [0, 1, 64])
def test_single_stream_decode_65536(splits):
    """Batch 1 x 65,536 keys, 16/2 heads: the split planner's extreme (two
    (sequence, KV head) units for 256 compute units); full output compared."""
    c = config_single_stream_decode()
    dc = DeviceCase(c)
    s = dc.calibrate()
    so = oracle_scales(c)
    assert s == so
    dc.store_all(s)
    out = dc.decode(s, num_splits=splits)
    torch.cuda.synchronize()
    kc, vc = oracle_cache(c, so)
    ref = paged_decode(c.q.float().numpy(), kc, vc, c.block_table, c.seq_lens, c.softmax_scale,
                       so["q"], so["k"], so["v"])
    print(check_attention(out, ref, "single-stream decode splits %d" % splits))


def test_local_prefill_q8192_sampled():
    """8,192 new tokens, window 512, 64/8 heads, learned bias of extent 128:
    the full launch, rows sampled at the window edges and at random."""
    c = config_local_prefill()
    dc = DeviceCase(c)
    s = dc.calibrate()
    so = oracle_scales(c)
    assert s == so
    dc.store_all(s)
    out = dc.prefill(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 511, 512, 513, 4095, 8191],
                                     rng.choice(8192, 40, replace=False)]))
    kc, vc = oracle_cache(c, so)
    ref = paged_prefill(c.q.float().numpy(), c.cu_q_lens, kc, vc, c.block_table, c.seq_lens,
                        c.softmax_scale, so["q"], so["k"], so["v"], c.window, None, rows=list(rows),
                        rel=c.rel)
    print(check_attention(out[torch.from_numpy(rows)], ref[rows], "local prefill q8192 w512"))


@pytest.mark.parametrize("hkv", [2, 8])
@pytest.mark.parametrize("n", [33, 2048, 16384])
def test_write_path_store_bit_exact(hkv, n):
    """Quant-on-store of the write-path sizes at 2 and 8 KV heads (the pages'
    model has 8 KV heads of 128 dims: TP1 and TP4 shares): cache bytes equal
    the oracle's store, with the calibrated scales and at v_scale 1.0 (the
    V outliers saturate)."""
    k, v, slot, num_pages = write_path_tokens(900 + hkv + n % 97, n, hkv)
    kn, vn = k.float().numpy(), v.float().numpy()
    for vs in (None, 1.0):
        ks = float(calibrate_amax(kn)[1])
        vsc = float(calibrate_amax(vn)[1]) if vs is None else vs
        cache = kvq.E4M3Cache(num_pages, hkv, 128)
        kvq.store(cache, k.cuda(), v.cuda(), torch.from_numpy(slot).cuda(), ks, vsc)
        torch.cuda.synchronize()
        kc, vc = new_cache(num_pages, hkv, 16, 128)
        store_e4m3(kc, vc, kn, vn, slot, ks, vsc)
        assert np.array_equal(cache.k.cpu().numpy(), kc)
        assert np.array_equal(cache.v.cpu().numpy(), vc)
