"""Host-side checks of the C ABI (no GPU needed, no kernel is launched):
the library loads, exports every function include/kvq.h declares, and
rejects bad arguments with the documented status before touching the GPU."""
import ctypes
import math
import os
import re

import pytest

import fp4_quantized_paged_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

FAKE = 0x100000  # a 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kvq.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kvq_store", "kvq_calibrate_amax", "kvq_paged_attn_decode",
            "kvq_paged_attn_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvq.h")).read()
    version = int(re.search(r"#define KVQ_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.kvq_abi_version() == version == kvq.ABI_VERSION
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert lib.kvq_status_str(s)
    assert lib.kvq_status_str(-6) != lib.kvq_status_str(-99)


def e4m3_desc(**kw):
    d = dict(format=1, page_size=16, num_kv_heads=4, head_dim=128, num_pages=64, k=FAKE, v=FAKE)
    d.update(kw)
    return kvq.CacheDesc(d["format"], d["page_size"], d["num_kv_heads"], d["head_dim"],
                         d["num_pages"], d["k"], d["v"])


def params(**kw):
    p = dict(num_q_heads=32, window=0, num_splits=0, rel_extent=0, softmax_scale=0.088,
             q_scale=1.0, k_scale=1.0, v_scale=1.0, alibi_slopes=None, rel_bias=None, flags=0)
    p.update(kw)
    return kvq.AttnParams(p["num_q_heads"], p["window"], p["num_splits"], p["rel_extent"],
                          p["softmax_scale"], p["q_scale"], p["k_scale"], p["v_scale"],
                          p["alibi_slopes"], p["rel_bias"], p["flags"])


def store(lib, desc, T=4, ks=1.0, vs=1.0, k=FAKE, v=FAKE, stride=512, slot=FAKE):
    return lib.kvq_store(ctypes.byref(desc), k, stride, v, stride, slot, T, ks, vs, None)


def test_store_validation(lib):
    assert lib.kvq_store(None, FAKE, 512, FAKE, 512, FAKE, 4, 1.0, 1.0, None) == -1
    assert store(lib, e4m3_desc(format=3)) == -2          # e.g. e5m2 / FNUZ: unknown format
    assert store(lib, e4m3_desc(format=0)) == -2
    assert store(lib, e4m3_desc(page_size=32)) == -2
    assert store(lib, e4m3_desc(head_dim=96)) == -2
    assert store(lib, e4m3_desc(k=None)) == -1
    assert store(lib, e4m3_desc(k=FAKE + 4)) == -1          # misaligned pool
    for bad in (0.0, -1.0, math.nan, math.inf):
        assert store(lib, e4m3_desc(), ks=bad) == -3
        assert store(lib, e4m3_desc(), vs=bad) == -3
    assert store(lib, e4m3_desc(), stride=500) == -1      # stride below one token
    assert store(lib, e4m3_desc(), stride=516) == -1      # not a multiple of 8
    assert store(lib, e4m3_desc(), T=-1) == -1
    assert store(lib, e4m3_desc(), slot=None) == -1
    assert store(lib, e4m3_desc(), T=0) == 0              # zero tokens: no launch
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert lib.kvq_store(ctypes.byref(nv), FAKE, 576, FAKE, 0, FAKE, 4, 1.0, 1.0, None) == -1
    assert lib.kvq_store(ctypes.byref(nv), FAKE, 576, None, 0, FAKE, 0, 1.0, 1.0, None) == 0
    assert lib.kvq_store(ctypes.byref(nv), FAKE, 576, None, 0, FAKE, 4, 0.0, 1.0, None) == -3
    bad_nv = kvq.CacheDesc(2, 16, 1, 512, 64, FAKE, None)
    assert lib.kvq_store(ctypes.byref(bad_nv), FAKE, 576, None, 0, FAKE, 4, 1.0, 1.0, None) == -2


def test_store_nvfp4_static_validation(lib):
    f = lib.kvq_store_nvfp4_static
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert f(None, FAKE, 576, FAKE, 4, 1.0, 1.0, None) == -1
    assert f(ctypes.byref(e4m3_desc()), FAKE, 576, FAKE, 4, 1.0, 1.0, None) == -2   # e4m3 pools: no
    assert f(ctypes.byref(kvq.CacheDesc(2, 16, 1, 512, 64, FAKE, None)), FAKE, 576, FAKE, 4, 1.0, 1.0, None) == -2
    for bad in (0.0, -1.0, math.nan, math.inf):
        assert f(ctypes.byref(nv), FAKE, 576, FAKE, 4, bad, 1.0, None) == -3      # RoPE scale
        assert f(ctypes.byref(nv), FAKE, 576, FAKE, 4, 1.0, bad, None) == -3      # outer scale
    assert f(ctypes.byref(nv), FAKE, 576, FAKE, -1, 1.0, 1.0, None) == -1
    assert f(ctypes.byref(nv), FAKE, 576, FAKE, 0, 1.0, 1.0, None) == 0          # no launch
    assert f(ctypes.byref(nv), None, 576, FAKE, 4, 1.0, 1.0, None) == -1
    assert f(ctypes.byref(nv), FAKE, 576, None, 4, 1.0, 1.0, None) == -1
    assert f(ctypes.byref(nv), FAKE + 8, 576, FAKE, 4, 1.0, 1.0, None) == -1      # misaligned input
    assert f(ctypes.byref(nv), FAKE, 570, FAKE, 4, 1.0, 1.0, None) == -1          # stride below a token
    assert f(ctypes.byref(nv), FAKE, 580, FAKE, 4, 1.0, 1.0, None) == -1          # stride % 8


def test_calibrate_validation(lib):
    f = lib.kvq_calibrate_amax
    assert f(FAKE, 10, 512, 512, None, None, None, None) == -1     # no amax buffer
    assert f(FAKE, 10, 500, 512, None, FAKE, None, None) == -1     # row_len % 8
    assert f(FAKE, 10, 512, 256, None, FAKE, None, None) == -1     # stride < row_len
    assert f(None, 10, 512, 512, None, FAKE, None, None) == -1
    assert f(FAKE + 2, 10, 512, 512, None, FAKE, None, None) == -1  # misaligned


def decode(lib, desc, p, B=2, max_len=100, ws=None, ws_bytes=0, bt_stride=64, q=FAKE):
    return lib.kvq_paged_attn_decode(ctypes.byref(desc), q, FAKE, bt_stride, FAKE, B, max_len,
                                     ctypes.byref(p), FAKE, ws, ws_bytes, None)


def test_decode_validation(lib):
    d = e4m3_desc()
    assert decode(lib, d, params(num_q_heads=30)) == -1          # Hq % Hkv != 0
    assert decode(lib, d, params(window=-1)) == -1
    assert decode(lib, d, params(rel_extent=1)) == -1                # extent without a table
    assert decode(lib, d, params(rel_bias=FAKE)) == -1               # table without an extent
    assert decode(lib, d, params(rel_bias=FAKE, rel_extent=(1 << 20) + 1)) == -1
    assert decode(lib, d, params(rel_bias=FAKE + 1, rel_extent=128)) == -1   # misaligned bf16
    assert decode(lib, d, params(rel_bias=FAKE, rel_extent=128, alibi_slopes=FAKE)) == -1
    assert decode(lib, d, params(rel_bias=FAKE, rel_extent=128), B=0) == 0
    assert decode(lib, d, params(flags=4)) == -1                     # unknown flag bit
    assert decode(lib, d, params(flags=3)) == -1                     # both P variants at once
    assert decode(lib, d, params(flags=2), B=0) == 0                 # the two-term prefill flag
    assert decode(lib, d, params(flags=1), B=0) == 0                 # the prefill flag: ignored here
    for bad in (0.0, -2.0, math.nan, math.inf):
        assert decode(lib, d, params(softmax_scale=bad)) == -3
        assert decode(lib, d, params(q_scale=bad)) == -3
        assert decode(lib, d, params(k_scale=bad)) == -3
        assert decode(lib, d, params(v_scale=bad)) == -3
    assert decode(lib, d, params(), B=0) == 0                    # no sequences: no launch
    assert decode(lib, d, params(), max_len=64 * 16 + 1) == -1   # table too short
    assert decode(lib, d, params(), q=FAKE + 2) == -1
    assert decode(lib, e4m3_desc(format=7), params()) == -2
    # forced splits need a workspace: too small -> KVQ_ERR_WORKSPACE
    p = params(num_splits=4)
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(d), 2, 1000, ctypes.byref(p))
    assert need == 2 * 32 * 4 * (128 + 2) * 4
    assert decode(lib, d, p, max_len=1000) == -4
    assert decode(lib, d, p, max_len=1000, ws=FAKE, ws_bytes=need - 4) == -4
    # one split needs none
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(d), 2, 1000, ctypes.byref(params(num_splits=1))) == 0


def decode_append(lib, desc, p, kn=FAKE, vn=FAKE, B=2, max_len=100, ws=None, ws_bytes=0):
    return lib.kvq_paged_attn_decode_append(ctypes.byref(desc), FAKE, kn, vn, FAKE, 64, FAKE, B, max_len,
                                            ctypes.byref(p), FAKE, ws, ws_bytes, None)


def test_decode_append_validation(lib):
    d = e4m3_desc()
    assert decode_append(lib, d, params(), kn=None) == -1
    assert decode_append(lib, d, params(), vn=None) == -1
    assert decode_append(lib, d, params(), kn=FAKE + 2) == -1        # not 16-byte aligned
    assert decode_append(lib, d, params(), vn=FAKE + 8) == -1
    for bad in (0.0, -1.0, math.nan, math.inf):
        assert decode_append(lib, d, params(k_scale=bad)) == -3
        assert decode_append(lib, d, params(v_scale=bad)) == -3
    assert decode_append(lib, d, params(), B=0) == 0                 # no sequences: no launch
    assert decode_append(lib, d, params(num_q_heads=30)) == -1
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert decode_append(lib, nv, params(num_q_heads=16)) == -2      # e4m3 only
    p = params(num_splits=4)
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(d), 2, 1000, ctypes.byref(p))
    assert decode_append(lib, d, p, max_len=1000, ws=FAKE, ws_bytes=need - 4) == -4


def test_decode_noalloc_validation(lib):
    """The no-alloc decode runs decode's host checks, then refuses a plan whose
    partials exceed the static scratch array; neither path launches."""
    f = lib.kvq_paged_attn_decode_noalloc
    d = e4m3_desc(num_pages=64 * 256)

    def call(p, B=2, max_len=100):
        return f(ctypes.byref(d), FAKE, FAKE, 256, FAKE, B, max_len, ctypes.byref(p), FAKE, None)

    assert call(params(num_q_heads=30)) == -1
    assert call(params(q_scale=0.0)) == -3
    assert call(params(), B=0) == 0
    assert call(params(), max_len=256 * 16 + 1) == -1          # table too short
    assert f(ctypes.byref(d), FAKE + 2, FAKE, 256, FAKE, 2, 100, ctypes.byref(params()), FAKE, None) == -1
    p = params(num_splits=32)
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(d), 64, 4096, ctypes.byref(p))
    assert need == 64 * 32 * 32 * (128 + 2) * 4 > kvq.NOALLOC_SCRATCH_BYTES
    assert call(p, B=64, max_len=4096) == -6
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert f(ctypes.byref(nv), FAKE, FAKE, 64, FAKE, 2, 100, ctypes.byref(params(num_q_heads=8)), FAKE,
             None) == -2


def test_nvfp4_decode_validation(lib):
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert decode(lib, nv, params(num_q_heads=8)) == -2                 # MLA decode takes 16 heads
    long_len = 64 * 512 * 16 + 1                                       # past 64 splits of 512 pages
    assert decode(lib, nv, params(num_q_heads=16), max_len=long_len, bt_stride=(long_len + 15) // 16) == -2
    assert decode(lib, nv, params(num_q_heads=16), B=0) == 0
    # no window or bias on the MLA path
    assert decode(lib, nv, params(num_q_heads=16, window=512), B=0) == -2
    assert decode(lib, nv, params(num_q_heads=16, alibi_slopes=FAKE), B=0) == -2
    assert decode(lib, nv, params(num_q_heads=16, rel_bias=FAKE, rel_extent=128), B=0) == -2


def test_prefill_validation(lib):
    d = e4m3_desc()
    f = lib.kvq_paged_attn_prefill
    p = params()
    assert f(ctypes.byref(d), FAKE, FAKE, 10, 5, FAKE, 64, FAKE, 2, 100, ctypes.byref(params(num_q_heads=31)),
             FAKE, None, 0, None) == -1
    assert f(ctypes.byref(d), FAKE, FAKE, 0, 0, FAKE, 64, FAKE, 2, 100, ctypes.byref(p), FAKE, None, 0, None) == 0
    assert f(ctypes.byref(d), FAKE, FAKE, 10, 200, FAKE, 64, FAKE, 2, 100, ctypes.byref(p), FAKE, None, 0,
             None) == -1                                        # max_q_len > max_seq_len
    # NVFP4 prefill: validation only (no call below reaches a launch)
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert f(ctypes.byref(nv), FAKE, FAKE, 10, 5, FAKE, 64, FAKE, 2, 100, ctypes.byref(params(num_q_heads=8)),
             FAKE, None, 0, None) == -2                           # 16 heads only
    assert f(ctypes.byref(nv), FAKE, FAKE, 10, 5, FAKE, 4096, FAKE, 2, 40000,
             ctypes.byref(params(num_q_heads=16)), FAKE, None, 0, None) == -2   # past 32,768 keys
    assert f(ctypes.byref(nv), FAKE, FAKE, 10, 5, FAKE, 64, FAKE, 2, 100,
             ctypes.byref(params(num_q_heads=16, window=64)), FAKE, None, 0, None) == -2
    assert f(ctypes.byref(nv), FAKE, FAKE, 0, 0, FAKE, 64, FAKE, 2, 100, ctypes.byref(params(num_q_heads=16)),
             FAKE, None, 0, None) == 0                            # no queries: no launch


def test_prefill_workspace_bytes(lib):
    """kvq_prefill_workspace_bytes: one fp32 key norm per (sequence, KV head,
    128-key block) with slopes on the e4m3 cache; 0 without slopes, for the
    NVFP4 format, for empty or invalid arguments."""
    d = e4m3_desc()
    q = lib.kvq_prefill_workspace_bytes
    assert q(ctypes.byref(d), 3, 1000, ctypes.byref(params(alibi_slopes=FAKE))) == 4 * 3 * 4 * 8
    assert q(ctypes.byref(d), 3, 1024, ctypes.byref(params(alibi_slopes=FAKE))) == 4 * 3 * 4 * 8
    assert q(ctypes.byref(d), 3, 1025, ctypes.byref(params(alibi_slopes=FAKE))) == 4 * 3 * 4 * 9
    assert q(ctypes.byref(d), 3, 1000, ctypes.byref(params())) == 0
    assert q(ctypes.byref(d), 0, 1000, ctypes.byref(params(alibi_slopes=FAKE))) == 0
    assert q(ctypes.byref(d), 3, 0, ctypes.byref(params(alibi_slopes=FAKE))) == 0
    assert q(ctypes.byref(d), 3, 1000, ctypes.byref(params(num_q_heads=31, alibi_slopes=FAKE))) == 0
    assert q(ctypes.byref(d), 3, 1000, None) == 0
    nv = kvq.CacheDesc(2, 16, 1, 576, 64, FAKE, None)
    assert q(ctypes.byref(nv), 3, 1000, ctypes.byref(params(num_q_heads=16))) == 0


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of kvq_cache and kvq_attn_params have the header's
    field offsets and sizes (checked by compiling offsetof/sizeof with gcc)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    structs = {"kvq_cache": kvq.CacheDesc, "kvq_attn_params": kvq.AttnParams}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "kvq.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append('  printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for fname, _ in cls._fields_:
            lines.append('  printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, fname, cname, fname))
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, field, val = line.split()
        got[(cname, field)] = int(val)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_calibration_extras_validation(lib):
    f = lib.kvq_scale_from_amax
    assert f(None, 0, FAKE, None) == -1
    assert f(FAKE, 0, None, None) == -1
    assert f(FAKE, 3, FAKE, None) == -1          # unknown rule
    assert f(FAKE, -1, FAKE, None) == -1
    g = lib.kvq_band_counts
    assert g(FAKE, 10, 512, 512, None, 1.0, None, None) == -1        # no counts buffer
    assert g(FAKE, 10, 512, 512, None, 1.0, FAKE + 4, None) == -1    # counts not 8-byte aligned
    assert g(FAKE, 10, 500, 512, None, 1.0, FAKE, None) == -1        # row_len % 8
    assert g(FAKE, 10, 512, 256, None, 1.0, FAKE, None) == -1        # stride < row_len
    for bad in (0.0, -1.0, math.nan, math.inf):
        assert g(FAKE, 10, 512, 512, None, bad, FAKE, None) == -3
    assert g(None, 10, 512, 512, None, 1.0, FAKE, None) == -1
    assert g(FAKE + 2, 10, 512, 512, None, 1.0, FAKE, None) == -1    # misaligned rows
    assert g(None, 0, 512, 512, None, 1.0, FAKE, None) == 0          # no rows: no launch
