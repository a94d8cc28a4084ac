"""GPU parity of the e4m3 chunked-prefill attention against the fp64 oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_paged_amd as kvq

from oracle.attention import paged_prefill
from workloads import config_chunked_prefill, make_attn_case, geometric_slopes
from parity import DeviceCase, oracle_scales, oracle_cache, seq_tokens, check_attention

pytestmark = pytest.mark.gpu


def run_case(c, rows=None, seqs=None, **kw):
    dc = DeviceCase(c)
    s = dc.calibrate()
    so = oracle_scales(c)
    assert s == so
    dc.store_all(s)
    out = dc.prefill(s, **kw)
    torch.cuda.synchronize()
    tok = None if seqs is None else seq_tokens(c, seqs)
    kc, vc = oracle_cache(c, so, tokens=tok)
    ref = paged_prefill(c.q.float().numpy(), c.cu_q_lens, kc, vc, c.block_table, c.seq_lens,
                        c.softmax_scale, so["q"], so["k"], so["v"], c.window, c.slopes, rows=rows,
                        rel=c.rel)
    if rows is not None:
        return dc, out[torch.from_numpy(np.asarray(rows))], ref[rows]
    return dc, out, ref


CASES = [
    # (seq_lens, q_lens, Hq, Hkv, window, slopes)
    ([137, 64, 501], [37, 64, 1], 32, 4, 0, True),
    ([137, 64, 501], [37, 64, 1], 32, 4, 0, False),
    ([300, 1000], [300, 33], 16, 2, 64, True),       # full prefill + sliding window
    ([777], [129], 8, 1, 0, True),                   # one KV head, group 8
    ([260, 90], [70, 90], 12, 3, 0, True),           # group 4: half the waves idle
    ([200], [45], 32, 2, 0, True),                   # group 16: two head blocks
    ([100, 50, 33], [0, 50, 0], 8, 2, 0, True),      # sequences without new tokens
    ([500, 40], [20, 7], 16, 2, 0, True),            # slope bias, one tile: 8 heads per workgroup
    ([300, 290], [256, 250], 16, 4, 0, True),        # slope bias, 8 tiles: one head per workgroup, key norms
    ([1200], [300], 8, 1, 100, True),                # slope bias, window, key norms
]


@pytest.mark.parametrize("lens,qlens,hq,hkv,window,bias", CASES)
def test_prefill_shapes(lens, qlens, hq, hkv, window, bias):
    slopes = geometric_slopes(hq) if bias else None
    c = make_attn_case("prefill", 200 + sum(qlens) + hq, lens, qlens, hq, hkv, 128,
                       v_std=2.0, window=window, slopes=slopes)
    _, out, ref = run_case(c)
    print(check_attention(out, ref, "prefill %s %s hq%d hkv%d w%d" % (lens, qlens, hq, hkv, window)))


REL_CASES = [
    # (seq_lens, q_lens, Hq, Hkv, window, extent): learned relative-bias table
    ([137, 64, 501], [37, 64, 1], 32, 4, 0, 128),
    ([300, 1000], [300, 33], 16, 2, 64, 128),        # sliding window at extent 128
    ([2600, 777], [129, 777], 8, 1, 0, 1024),         # far blocks and near blocks
    ([260, 90], [70, 90], 12, 3, 0, 1),
    ([900], [45], 32, 2, 0, 4096),                    # extent past every distance
]


@pytest.mark.parametrize("lens,qlens,hq,hkv,window,extent", REL_CASES)
def test_prefill_learned_bias(lens, qlens, hq, hkv, window, extent):
    c = make_attn_case("prefill_rel", 400 + sum(qlens) + hq, lens, qlens, hq, hkv, 128,
                       v_std=2.0, window=window, rel_extent=extent)
    _, out, ref = run_case(c)
    print(check_attention(out, ref, "prefill rel %s %s hq%d w%d E%d" % (lens, qlens, hq, window, extent)))


def test_chunked_prefill_full_size_sampled():
    """4 x (32,768 cached + 2,048 new) tokens, 32/4 heads: the whole launch
    runs; 3 x 40 sampled query rows (first, last, ragged positions) are
    compared against the oracle."""
    c = config_chunked_prefill()
    rng = np.random.default_rng(0)
    rows = []
    for b in (0, 2, 3):
        r0 = int(c.cu_q_lens[b])
        picks = np.concatenate([[0, 1, 31, 32, 2047], rng.choice(2048, 35, replace=False)])
        rows += list(r0 + np.unique(picks))
    _, out, ref = run_case(c, rows=rows, seqs=[0, 2, 3])
    print(check_attention(out, ref, "chunked_prefill"))


def test_prefill_poisoned_pool_and_determinism():
    c = make_attn_case("ppoison", 41, [70, 33, 16], [70, 20, 3], 16, 2, 128, spare_frac=2.0,
                       slopes=geometric_slopes(16))
    dc = DeviceCase(c, fill=0x7F)
    s = dc.calibrate()
    dc.store_all(s)
    a = dc.prefill(s)
    b = dc.prefill(s)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(a.float()))
    assert torch.equal(a, b)


def check_fp8_p(out, ref, label):
    """The single-term e4m3 P variant against the exact oracle: within the
    pages' fp8 attention test tolerance, atol = rtol = 0.15 (vLLM PR 54705,
    "Test Plan"), elementwise. Returns the measured errors."""
    o = out.float().cpu().numpy().astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(o - r)
    bad = err > 0.15 + 0.15 * np.abs(r)
    assert not bad.any(), (label, np.argwhere(bad)[:5])
    assert np.all(np.isfinite(o))
    return {"max_abs": float(err.max()), "rel_l2": float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-30))}


FP8P_CASES = [
    # (seq_lens, q_lens, Hq, Hkv, window, bias): bias None / "slopes" / extent
    ([137, 64, 501], [37, 64, 1], 32, 4, 0, "slopes"),
    ([137, 64, 501], [37, 64, 1], 32, 4, 0, None),
    ([300, 1000], [300, 33], 16, 2, 64, "slopes"),
    ([2600, 777], [129, 777], 8, 1, 0, 1024),
    ([100, 50, 33], [0, 50, 0], 8, 2, 0, "slopes"),
]


@pytest.mark.parametrize("lens,qlens,hq,hkv,window,bias", FP8P_CASES)
def test_prefill_fp8_p_variant(lens, qlens, hq, hkv, window, bias):
    kw = {}
    if bias == "slopes":
        kw["slopes"] = geometric_slopes(hq)
    elif bias is not None:
        kw["rel_extent"] = bias
    c = make_attn_case("prefill_p8", 500 + sum(qlens) + hq, lens, qlens, hq, hkv, 128,
                       v_std=2.0, window=window, **kw)
    dc, out, ref = run_case(c, fp8_p=True)
    print(check_fp8_p(out, ref, "fp8 P %s %s w%d %s" % (lens, qlens, window, bias)))
    s = dc.calibrate()
    again = dc.prefill(s, fp8_p=True)
    torch.cuda.synchronize()
    assert torch.equal(again, out)


@pytest.mark.parametrize("lens,qlens,hq,hkv,window,bias", FP8P_CASES)
def test_prefill_fp8_p2_variant(lens, qlens, hq, hkv, window, bias):
    """Two e4m3 terms of P on fp8 MFMA: the default tolerance applies."""
    kw = {}
    if bias == "slopes":
        kw["slopes"] = geometric_slopes(hq)
    elif bias is not None:
        kw["rel_extent"] = bias
    c = make_attn_case("prefill_p82", 600 + sum(qlens) + hq, lens, qlens, hq, hkv, 128,
                       v_std=2.0, window=window, **kw)
    dc, out, ref = run_case(c, fp8_p2=True)
    print(check_attention(out, ref, "fp8 P x2 %s %s w%d %s" % (lens, qlens, window, bias)))


def test_chunked_prefill_fp8_p2_full_size_sampled():
    c = config_chunked_prefill()
    rng = np.random.default_rng(2)
    rows = []
    for b in (0, 2):
        r0 = int(c.cu_q_lens[b])
        picks = np.concatenate([[0, 2047], rng.choice(2048, 30, replace=False)])
        rows += list(r0 + np.unique(picks))
    _, out, ref = run_case(c, rows=rows, seqs=[0, 2], fp8_p2=True)
    print(check_attention(out, ref, "chunked_prefill fp8 P x2"))


def test_chunked_prefill_fp8_p_full_size_sampled():
    c = config_chunked_prefill()
    rng = np.random.default_rng(1)
    rows = []
    for b in (1, 3):
        r0 = int(c.cu_q_lens[b])
        picks = np.concatenate([[0, 2047], rng.choice(2048, 30, replace=False)])
        rows += list(r0 + np.unique(picks))
    _, out, ref = run_case(c, rows=rows, seqs=[1, 3], fp8_p=True)
    print(check_fp8_p(out, ref, "chunked_prefill fp8 P"))


def slope_table(slopes, extent):
    """The slope bias written out as a learned table: T[h][d] = bf16(fp32(slope_h) * fp32(-d))."""
    d = -np.arange(extent, dtype=np.float32)
    prod = (np.asarray(slopes, dtype=np.float32)[:, None] * d[None, :]).astype(np.float32)
    return torch.from_numpy(prod).to(torch.bfloat16)


@pytest.mark.parametrize("pmode", ["f16", "fp8_p", "fp8_p2"])
@pytest.mark.parametrize("which", ["small", "full"])
def test_prefill_slope_early_stop_is_exact(which, pmode):
    """With the slope bias a wave stops once a bound puts every remaining
    probability at exactly zero, and both bias kinds skip blocks whose every P
    is zero. The learned-table path, given a table holding the same bf16
    biases with an extent past every distance, never stops early: the two
    outputs are equal bit for bit, on a small case and on the full
    4 x (32,768 + 2,048) launch."""
    if which == "full":
        c = config_chunked_prefill()
    else:
        c = make_attn_case("pstop", 77, [4096, 3000, 700], [200, 77, 700], 32, 4, 128,
                           v_std=2.0, slopes=geometric_slopes(32))
    dc = DeviceCase(c)
    s = dc.calibrate()
    dc.store_all(s)
    mode = {} if pmode == "f16" else {pmode: True}
    a = dc.prefill(s, **mode)
    tab = slope_table(c.slopes, c.max_seq_len).cuda()
    b = kvq.prefill(dc.cache, dc.q, dc.cu_q_lens, c.max_q_len, dc.block_table, dc.seq_lens,
                    c.max_seq_len, c.softmax_scale, s["q"], s["k"], s["v"], c.window, None,
                    rel_bias=tab, **mode)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(a.float()))
    assert torch.equal(a, b)


def far_live_case():
    """A key that outscores every other by far, planted 3,800+ positions behind
    the new tokens: under a slope of 0.05 per position the blocks between it
    and the diagonal hold only probabilities that round to zero and are
    skipped, and the planted key's block, far out, must not be. Every query
    has +5 on dim 0 and the planted key is 3,000 e_0."""
    c = make_attn_case("farlive", 91, [4096, 700], [64, 40], 8, 1, 128,
                       slopes=np.full(8, 0.05, dtype=np.float32))
    q = c.q.float()
    q[:, :, 0] += 5.0
    c.q = q.to(torch.bfloat16)
    k = c.k.float()
    planted = int(np.nonzero((c.seq_of_token == 0) & (c.pos_of_token == 200))[0][0])
    k[planted] = 0.0
    k[planted, 0, 0] = 3000.0
    c.k = k.to(torch.bfloat16)
    return c


@pytest.mark.parametrize("pmode", ["f16", "fp8_p2"])
def test_prefill_far_live_block_after_skipped_blocks(pmode):
    """The block holding the planted key is needed for PV although many blocks
    before it were skipped (and the slope path's early stop must not fire
    before it). Checked against the oracle, and bit for bit against the
    learned-table path given the same biases."""
    c = far_live_case()
    mode = {} if pmode == "f16" else {pmode: True}
    dc, out, ref = run_case(c, **mode)
    print(check_attention(out, ref, "far live block %s" % pmode))
    s = dc.calibrate()
    tab = slope_table(c.slopes, c.max_seq_len).cuda()
    b = kvq.prefill(dc.cache, dc.q, dc.cu_q_lens, c.max_q_len, dc.block_table, dc.seq_lens,
                    c.max_seq_len, c.softmax_scale, s["q"], s["k"], s["v"], c.window, None,
                    rel_bias=tab, **mode)
    torch.cuda.synchronize()
    assert torch.equal(out, b)


def test_prefill_key_norm_workspace():
    """The slope-bias prefill's key-norm pass (white box): for every
    (sequence, KV head, 128-key block) the workspace holds the largest
    Euclidean norm of the block's stored key codes over keys before the
    sequence end, never below the exact value (fp64 over the oracle's store)
    and above it by at most 2e-4 relative. The output equals the one computed
    without the workspace (the looser 448 * sum |q| bound) bit for bit."""
    from oracle.codecs import e4m3_decode
    c = make_attn_case("knorm", 78, [4096, 3000, 700], [300, 77, 700], 32, 4, 128,
                       v_std=2.0, slopes=geometric_slopes(32))
    dc = DeviceCase(c)
    s = dc.calibrate()
    dc.store_all(s)
    B, G = len(c.seq_lens), c.num_kv_heads
    nblk = (c.max_seq_len + 127) // 128
    need = kvq.prefill_workspace_bytes(dc.cache, B, c.max_seq_len, c.num_q_heads, slopes=dc.slopes)
    assert need == 4 * B * G * nblk
    assert kvq.prefill_workspace_bytes(dc.cache, B, c.max_seq_len, c.num_q_heads) == 0   # no slopes
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    a = dc.prefill(s, workspace=ws)
    b = dc.prefill(s, use_workspace=False)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(a.float()))
    assert torch.equal(a, b)
    got = ws.view(torch.float32).cpu().numpy().reshape(B, G, nblk)
    kc, _ = oracle_cache(c, oracle_scales(c))
    for bi, L in enumerate(c.seq_lens.tolist()):
        pos = np.arange(L)
        pages = c.block_table[bi][pos // 16]
        for g in range(G):
            codes = kc[pages, g, pos % 16, :]
            norm = np.sqrt((e4m3_decode(codes).astype(np.float64) ** 2).sum(-1))
            nb = (L + 127) // 128
            want = np.array([norm[j * 128:(j + 1) * 128].max() for j in range(nb)])
            have = got[bi, g, :nb].astype(np.float64)
            assert np.all(have >= want), (bi, g, np.argmin(have - want))
            assert np.all(have <= want * (1 + 2e-4)), (bi, g)


@pytest.mark.parametrize("nq", [64, 300])
def test_prefill_far_live_block_with_key_norms(nq):
    """The planted far key (far_live_case) with enough new tokens for the
    key-norm pass (nq = 300) and without (nq = 64): its block's norm keeps
    the early stop from firing above it; oracle parity and bit-equality with
    the call that takes no workspace."""
    c = make_attn_case("farlive_n", 92, [4096, 700], [nq, 40], 8, 1, 128,
                       slopes=np.full(8, 0.05, dtype=np.float32))
    q = c.q.float()
    q[:, :, 0] += 5.0
    c.q = q.to(torch.bfloat16)
    k = c.k.float()
    planted = int(np.nonzero((c.seq_of_token == 0) & (c.pos_of_token == 200))[0][0])
    k[planted] = 0.0
    k[planted, 0, 0] = 3000.0
    c.k = k.to(torch.bfloat16)
    dc, out, ref = run_case(c)
    print(check_attention(out, ref, "far live block, %d new tokens" % nq))
    s = dc.calibrate()
    b = dc.prefill(s, use_workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(out, b)


def test_prefill_key_norms_poisoned_pool():
    """Pages past every sequence end poisoned with e4m3 NaN codes, slope bias,
    enough new tokens for the key-norm pass: outputs finite, deterministic and
    equal to the call without the workspace."""
    c = make_attn_case("kpoison", 43, [700, 300, 16], [300, 280, 3], 16, 2, 128, spare_frac=2.0,
                       slopes=geometric_slopes(16))
    dc = DeviceCase(c, fill=0x7F)
    s = dc.calibrate()
    dc.store_all(s)
    a = dc.prefill(s)
    b = dc.prefill(s)
    n = dc.prefill(s, use_workspace=False)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(a.float()))
    assert torch.equal(a, b) and torch.equal(a, n)
