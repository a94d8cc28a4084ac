"""The no-alloc decode entry point (kvq_paged_attn_decode_noalloc): its split
partials live in the library's static scratch array instead of a caller
workspace. Through the C ABI, two calls in a row (the second smaller) must
give the same output bits as kvq_paged_attn_decode with a workspace, for the
e4m3 and the NVFP4 caches, with the split plan that uses the scratch."""
import numpy as np
import pytest
import torch

import fp4_quantized_paged_amd as kvq
from workloads import make_attn_case, make_mla_case, geometric_slopes
from parity import DeviceCase, oracle_scales

pytestmark = pytest.mark.gpu


def e4m3_pair(case, splits, slopes=True):
    dc = DeviceCase(case)
    s = oracle_scales(case)
    dc.store_all(s)
    c = case
    args = (dc.cache, dc.q, dc.block_table, dc.seq_lens, c.max_seq_len, c.softmax_scale, s["q"], s["k"],
            s["v"], c.window, dc.slopes)
    need = kvq.decode_workspace_bytes(dc.cache, c.batch, c.max_seq_len, dc.q.shape[1], c.window, splits)
    assert 0 < need <= kvq.NOALLOC_SCRATCH_BYTES, need
    ref = kvq.decode(*args, num_splits=splits)
    out = torch.full_like(ref, float("nan"))
    got = kvq.decode_noalloc(*args, num_splits=splits, out=out)
    torch.cuda.synchronize()
    return got, ref, need


def test_noalloc_e4m3_two_calls():
    big = make_attn_case("noalloc_big", 901, [20000, 9000, 17, 4097], [1] * 4, 32, 4, 128,
                         qk_dist="rms20", v_std=4.0, v_outlier_frac=1e-3, slopes=geometric_slopes(32))
    got, ref, need_big = e4m3_pair(big, 0)
    assert torch.equal(got, ref)
    small = make_attn_case("noalloc_small", 902, [3000, 700], [1] * 2, 8, 2, 64,
                           qk_dist="rms20", v_std=4.0, v_outlier_frac=1e-3, window=500)
    got, ref, need_small = e4m3_pair(small, 3)
    assert need_small < need_big
    assert torch.equal(got, ref)


def mla_pair(case, splits):
    cache = kvq.Nvfp4Cache(case.num_pages)
    kvq.store(cache, case.kv.cuda(), None, torch.from_numpy(case.slot_mapping).cuda(), case.rope_scale)
    q = case.q.cuda()
    bt = torch.from_numpy(case.block_table).cuda()
    sl = torch.from_numpy(case.seq_lens).cuda()
    need = kvq.decode_workspace_bytes(cache, case.batch, case.max_seq_len, 16, 0, splits)
    assert 0 < need <= kvq.NOALLOC_SCRATCH_BYTES, need
    ref = kvq.decode(cache, q, bt, sl, case.max_seq_len, case.softmax_scale, k_scale=case.rope_scale,
                     num_splits=splits)
    out = torch.full_like(ref, float("nan"))
    got = kvq.decode_noalloc(cache, q, bt, sl, case.max_seq_len, case.softmax_scale, k_scale=case.rope_scale,
                             num_splits=splits, out=out)
    torch.cuda.synchronize()
    return got, ref, need


def test_noalloc_nvfp4_two_calls():
    big = make_mla_case("noalloc_mla_big", 903, [8192, 5000, 1, 4096], layer_std=1.0)
    got, ref, need_big = mla_pair(big, 0)
    assert torch.equal(got, ref)
    small = make_mla_case("noalloc_mla_small", 904, [1000, 300], layer_std=0.05)
    got, ref, need_small = mla_pair(small, 3)
    assert need_small < need_big
    assert torch.equal(got, ref)


def test_noalloc_rejects_oversize_partials():
    """A plan whose partials exceed the static array is refused before any
    launch, and the output is left untouched."""
    B, L, hq = 64, 4096, 32
    cache = kvq.E4M3Cache(B * L // 16, 4, 128, fill=0)
    q = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.arange(B * L // 16, dtype=torch.int32, device="cuda").reshape(B, L // 16)
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    need = kvq.decode_workspace_bytes(cache, B, L, hq, 0, 32)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_noalloc(cache, q, bt, sl, L, 0.088, num_splits=32, out=out)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
