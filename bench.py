"""Benchmark of the quantized-KV-cache attention path on one MI355X.

A step is one decode step of the batched-decode workload (batch 64, 8,192-token
context, 32 query / 4 KV heads, head_dim 128, 16-token pages): quant-on-store
of the 64 new tokens' K/V into the paged e4m3 cache, then fp8 paged decode
attention over the full context (Q quantization, split-KV attention, combine).
Scales come from amax calibration over the resident inputs before timing.

``value`` is the step's algorithmic HBM bytes divided by the step time (GB/s).
The JSON line also carries the roofline of the dominant kernel (decode attention,
timed with HIP events on the launch stream), the other rows of the path measured
in the same run (stores, calibration, long-context and single-stream decode,
chunked and sliding-window prefill, NVFP4 record store, MLA decode and prefill),
and the CPU oracle timed on a bounded sample as a baseline.

Every row is timed the same way: 5 warm-up calls, then 20 groups of a few
back-to-back calls, each group between one pair of HIP events on the launch
stream; a row reports the median and the minimum of the per-call times over
the groups, a roofline object (algorithmic bytes or flops per call over the
median time, against the MI355X peak of the unit that bounds it) and the
SHA-256 of its inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-extras]
       [--skip-cpu] [--only ROW] [--copy-probe]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
FP8_PEAK_TFLOPS = 5000.0        # dense fp8 MFMA
FP16_PEAK_TFLOPS = 2500.0       # dense fp16 / bf16 MFMA
# e4m3 prefill: QK^T on fp8 MFMA and PV on fp16 MFMA, half the flops each:
# the time at peak is F/2 / 5000 + F/2 / 2500, i.e. a mixed peak of 3333 TFLOP/s
PREFILL_MIXED_PEAK_TFLOPS = 1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / FP16_PEAK_TFLOPS)
REPS = 20            # timed groups per row
WARM = 5             # warm-up calls per row


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--skip-extras", action="store_true", help="only the headline step")
    ap.add_argument("--skip-cpu", action="store_true", help="no CPU oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--only", choices=["prefill", "long_context", "nvfp4", "nvfp4_prefill", "tier1", "stores",
                                       "mla_decode"], default=None,
                    help="run only these rows (for profiling); prints their JSON")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class EventTimer:
    """Accumulates kernel time between HIP events recorded on torch's current
    stream (the stream the library launches on).

    The events are timing-only (hipEventDisableSystemFence): recording one
    skips the system-scope release, whose cache writeback and invalidate
    otherwise add several microseconds around every timed launch and push the
    next kernel back. They are created through the HIP runtime that torch has
    already loaded (libamdhip64.so.7 resolves to that same library)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with HIP error %d" % (what, rc))

    def _record(self):
        e = self.ct.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        stream = self.torch.cuda.current_stream().cuda_stream
        self._check(self.hip.hipEventRecord(e, self.ct.c_void_p(stream)), "hipEventRecord")
        return e

    def start(self):
        return self._record()

    def stop(self, s):
        self.pairs.append((s, self._record()))

    def mean_ms(self):
        if not self.pairs:
            return 0.0
        self._check(self.hip.hipEventSynchronize(self.pairs[-1][1]), "hipEventSynchronize")
        total = 0.0
        ms = self.ct.c_float()
        for a, b in self.pairs:
            self._check(self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
            total += ms.value
        n = len(self.pairs)
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        self.pairs = []
        return total / n


def decode_bytes(B, Hq, Hkv, D, L):
    """Algorithmic HBM bytes of one decode call: K and V codes of every attended
    token, bf16 Q in and bf16 O out, block table and lengths."""
    kv = B * L * Hkv * D * 2
    return kv + B * Hq * D * 2 * 2 + B * ((L + 15) // 16) * 4 + B * 4


def store_bytes(T, Hkv, D):
    """bf16 K and V in, e4m3 K and V out, one int64 slot per token."""
    return T * (Hkv * D * (2 * 2 + 2) + 8)


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "decode_e4m3_batched_decode.md")


def traffic_record():
    """HBM traffic per launch of the decode kernel from the committed rocprofv3
    counter summary, or None when the kernel sources changed since the
    counters were taken (their SHA-256 no longer matches)."""
    import hashlib
    try:
        line = [l for l in open(TRAFFIC_PROFILE) if l.startswith("traffic_record: ")][0]
        rec = json.loads(line[len("traffic_record: "):])
        root = os.path.dirname(os.path.abspath(__file__))
        h = hashlib.sha256()
        for f in rec["kernel_sources"]:
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest() != rec["kernel_sources_sha256"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, IndexError, KeyError, ValueError):
        return None


def copy_probe(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "note": "one copy kernel reads and writes n bytes"}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X "
              "(no collectives or sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(torch)
        return
    import fp4_quantized_paged_amd as kvq
    from workloads import config_batched_decode

    kvq.lib()   # fail loudly when the HIP library is missing
    torch.cuda.set_device(0)
    if args.only is not None:
        fn = {"prefill": prefill_rows, "long_context": long_context_rows, "nvfp4": nvfp4_rows,
              "nvfp4_prefill": nvfp4_prefill_rows, "tier1": tier1_rows, "stores": write_path_rows,
              "mla_decode": mla_decode_only}[args.only]
        print(json.dumps(fn(torch, kvq)), flush=True)
        return
    dev = "cuda"

    # ---------------- headline: batched decode step ----------------
    log("generating batched-decode inputs")
    c = config_batched_decode()
    sha = case_sha(c)
    B, Hq, Hkv, D, L = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.max_seq_len
    k = c.k.to(dev)
    v = c.v.to(dev)
    q = c.q.to(dev)
    slot = torch.from_numpy(c.slot_mapping).to(dev)
    bt = torch.from_numpy(c.block_table).to(dev)
    seq_lens = torch.from_numpy(c.seq_lens).to(dev)
    _, ks = kvq.calibrate_amax(k)
    _, qs = kvq.calibrate_amax(q)
    scales = {"k": float(ks.item()), "q": float(qs.item()), "v": float(c.v_scale_override)}
    # two cache copies (1 GiB together) alternate between steps so the 256 MB
    # Infinity Cache cannot serve the KV reads of one step from the last
    caches = [kvq.E4M3Cache(c.num_pages, Hkv, D) for _ in range(2)]
    for cache in caches:
        kvq.store(cache, k, v, slot, scales["k"], scales["v"])
    new_idx = torch.from_numpy(np.cumsum(c.seq_lens) - 1).to(dev)   # current token of each seq
    k_new = k[new_idx].contiguous()
    v_new = v[new_idx].contiguous()
    slot_new = slot[new_idx].contiguous()
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ws_bytes = kvq.decode_workspace_bytes(caches[0], B, L, Hq)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def decode(i):
        kvq.decode(caches[i % 2], q, bt, seq_lens, L, c.softmax_scale, scales["q"], scales["k"],
                   scales["v"], out=out, workspace=ws)

    def step(i):
        # the current tokens' quant-on-store and the decode in one launch
        kvq.decode(caches[i % 2], q, bt, seq_lens, L, c.softmax_scale, scales["q"], scales["k"],
                   scales["v"], out=out, workspace=ws, k_new=k_new, v_new=v_new)

    def step_unfused(i):
        kvq.store(caches[i % 2], k_new, v_new, slot_new, scales["k"], scales["v"])
        decode(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    dec_bytes = decode_bytes(B, Hq, Hkv, D, L)
    step_bytes = dec_bytes + store_bytes(B, Hkv, D)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # Decode kernel time for the roofline: the same decode launches back to
    # back (same alternating caches), between one pair of HIP events on the
    # launch stream, so that no event sits between two launches.
    dec_ms = back_to_back_ms(torch, decode, args.steps)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9
    # the same step as two launches (kvq_store, then kvq_paged_attn_decode)
    unfused_ms = back_to_back_ms(torch, step_unfused, args.steps)
    result = {
        "metric": "fp8 paged-decode attention HBM GB/s & % of peak; KV store tokens/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic (seeded; Q/K RMS-normed amax 20, V std 8 with 0.1% outliers in [448, 1272])",
        "config": {"workload": "batched_decode", "batch": B, "context": L, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "page_size": 16, "kv_format": "e4m3",
                   "scales": scales,
                   "step": "store 64 new tokens + decode attention, one launch (kvq_paged_attn_decode_append)"},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "kernel": "decode_e4m3_kernel (batched decode)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_record(),
                     "bytes_per_launch": dec_bytes, "avg_launch_us": round(dec_ms * 1e3, 2)},
        "inputs_sha256": sha,
        "step_unfused_us": round(unfused_ms * 1e3, 2),
    }
    log("decode %.2f us, %.0f GB/s (%.1f%% of peak)" % (dec_ms * 1e3, achieved,
                                                         100 * achieved / HBM_PEAK_GBPS))
    rel_rows = {}
    if not args.skip_extras:
        # the same decode with a learned relative-bias table of 1,024 entries
        from workloads import rel_bias_table
        rel = torch.from_numpy(rel_bias_table(np.random.default_rng(5), Hq, 1024)).to(torch.bfloat16).to(dev)

        def decode_rel(i):
            kvq.decode(caches[i % 2], q, bt, seq_lens, L, c.softmax_scale, scales["q"], scales["k"],
                       scales["v"], out=out, workspace=ws, rel_bias=rel)
        rel_rows["decode_rel1024"] = timed_row(torch, decode_rel, "hbm", dec_bytes, HBM_PEAK_GBPS, "GB/s",
                                               per=5, sha=sha)
        rel_rows["decode"] = timed_row(torch, decode, "hbm", dec_bytes, HBM_PEAK_GBPS, "GB/s", per=5, sha=sha,
                                       roof_extra={"kernel": "decode_e4m3_kernel"})
    del caches, k_new, v_new

    if not args.skip_extras:
        result["rows"] = extras(torch, kvq, c, k, v, q, slot, scales, sha)
        result["rows"].update(rel_rows)
    del k, v, q
    torch.cuda.empty_cache()

    if not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(result), flush=True)


PRIMER_CYCLES = 4_000_000   # a GPU spin of ~2 ms: longer than the host needs to queue 20 calls


def back_to_back_ms(torch, fn, reps):
    """Mean GPU time of reps back-to-back calls fn(0 .. reps-1) between one pair
    of HIP events. A spin kernel queued first keeps the GPU busy while the host
    queues the start event and the calls, so neither host launch time nor idle
    GPU time falls between the events."""
    t = EventTimer(torch)
    torch.cuda._sleep(PRIMER_CYCLES)
    s = t.start()
    for i in range(reps):
        fn(i)
    t.stop(s)
    return t.mean_ms() / reps


def timed_stats(torch, fn, per=5, reps=REPS, warm=WARM):
    """Per-call GPU time of fn(i) in microseconds: WARM warm-up calls, then
    REPS groups of `per` back-to-back calls, each group between one pair of
    HIP events. Returns (median, min) over the groups. The call index i keeps
    counting across groups, so callers that alternate buffers by i do."""
    for i in range(warm):
        fn(i)
    base = [warm]
    samples = []
    for _ in range(reps):
        off = base[0]
        samples.append(back_to_back_ms(torch, lambda j: fn(off + j), per) * 1e3)
        base[0] += per
    return float(np.median(samples)), float(np.min(samples))


def roofline(bound, amount, us, peak, unit, **extra):
    """Roofline record of one call: `amount` algorithmic bytes (unit GB/s) or
    flops (TFLOP/s) over `us` microseconds against `peak`."""
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = amount / (us * 1e-6) / scale
    rec = {"bound": bound, "achieved": round(achieved, 1), "peak": round(peak, 1), "unit": unit,
           "frac": round(achieved / peak, 4), ("bytes" if unit == "GB/s" else "flops"): int(amount)}
    rec.update(extra)
    return rec


def timed_row(torch, fn, bound, amount, peak, unit, per=5, sha=None, roof_extra=None, **fields):
    """One bench row: median / min per-call time and the roofline at the median."""
    med, mn = timed_stats(torch, fn, per=per)
    row = dict(fields)
    row.update({"us_median": round(med, 2), "us_min": round(mn, 2), "reps": REPS, "calls_per_rep": per,
                "roofline": roofline(bound, amount, med, peak, unit, **(roof_extra or {}))})
    if sha is not None:
        row["inputs_sha256"] = sha
    return row


def sha256_of(*arrays):
    """SHA-256 over the bytes of the given host arrays / CPU tensors, in order."""
    import hashlib
    import torch
    h = hashlib.sha256()
    for a in arrays:
        if a is None:
            continue
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous().reshape(-1).view(torch.uint8).numpy()
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def case_sha(c):
    """SHA-256 of an attention workload's inputs (Q, K, V, slots, block table,
    lengths, new-token counts, slopes or bias table)."""
    return sha256_of(c.q, c.k, c.v, c.slot_mapping, c.block_table, c.seq_lens, c.cu_q_lens, c.slopes, c.rel)


def mla_sha(c):
    return sha256_of(c.q, c.kv, c.slot_mapping, c.block_table, c.seq_lens)


def extras(torch, kvq, c, k, v, q, slot, scales, sha):
    """Other rows of the path on the batched-decode inputs, then the other
    workloads' rows."""
    rows = {}
    Hkv, D = c.num_kv_heads, c.head_dim
    T = k.shape[0]
    # bulk quant-on-store of all 524,288 tokens (1 GiB of bf16 read per call)
    cache = kvq.E4M3Cache(c.num_pages, Hkv, D)
    sb = store_bytes(T, Hkv, D)
    rows["store_bulk"] = timed_row(torch, lambda i: kvq.store(cache, k, v, slot, scales["k"], scales["v"]),
                                   "hbm", sb, HBM_PEAK_GBPS, "GB/s", per=2, sha=sha, tokens=T,
                                   kv_heads=Hkv)
    rows["store_bulk"]["tokens_per_s"] = round(T / (rows["store_bulk"]["us_median"] * 1e-6), 1)
    # decode append: the 64 new tokens only (latency-bound)
    idx = torch.from_numpy(np.cumsum(c.seq_lens) - 1).to(k.device)
    kn, vn, sn = k[idx].contiguous(), v[idx].contiguous(), slot[idx].contiguous()
    rows["store_append"] = timed_row(torch, lambda i: kvq.store(cache, kn, vn, sn, scales["k"], scales["v"]),
                                     "hbm", store_bytes(64, Hkv, D), HBM_PEAK_GBPS, "GB/s", per=10, sha=sha,
                                     tokens=int(kn.shape[0]), note="latency-bound")
    # calibration over K and V (2 bytes read per element)
    amax = torch.zeros(1, device=k.device)
    cb = 2 * k.numel() * 2
    rows["calibrate_kv"] = timed_row(torch, lambda i: (kvq.calibrate_amax(k, amax=amax),
                                                       kvq.calibrate_amax(v, amax=amax)),
                                     "hbm", cb, HBM_PEAK_GBPS, "GB/s", per=2, sha=sha)
    # clip / flush-to-zero band counters of K and V at their scales
    counts = torch.zeros(2, dtype=torch.int64, device=k.device)
    rows["band_counts_kv"] = timed_row(torch, lambda i: (kvq.band_counts(k, scales["k"], counts=counts),
                                                         kvq.band_counts(v, scales["v"], counts=counts)),
                                       "hbm", cb, HBM_PEAK_GBPS, "GB/s", per=2, sha=sha)
    del cache
    torch.cuda.empty_cache()
    rows.update(write_path_rows(torch, kvq))
    rows.update(tiny_decode_rows(torch, kvq))
    rows.update(long_context_rows(torch, kvq))
    rows.update(tier1_rows(torch, kvq))
    rows.update(prefill_rows(torch, kvq))
    rows.update(nvfp4_rows(torch, kvq))
    return rows


def write_path_rows(torch, kvq):
    """The write path of the vLLM PR 54705 evidence document ("Tier 1": 2 head
    configurations x {sliding, global} x {33, 2,048, 16,384} tokens). The
    pages' model has 8 KV heads of 128 dims, 2 per rank at TP4: rows at 2, 4
    (the batched-decode shape) and 8 KV heads. A sliding-window layer stores
    its tokens with the same call as a global one (the window only decides
    which pages a caller keeps), so one row covers both."""
    from workloads import write_path_tokens
    log("write path")
    out = {}
    dev = "cuda"
    for hkv in (2, 4, 8):
        for n in (33, 2048, 16384):
            k, v, slot, num_pages = write_path_tokens(900 + hkv + n % 97, n, hkv)
            sha = sha256_of(k, v, slot)
            kd, vd, sd = k.to(dev), v.to(dev), torch.from_numpy(slot).to(dev)
            cache = kvq.E4M3Cache(num_pages, hkv, 128)
            r = timed_row(torch, lambda i: kvq.store(cache, kd, vd, sd, 0.05, 3.0), "hbm",
                          store_bytes(n, hkv, 128), HBM_PEAK_GBPS, "GB/s", per=10, sha=sha,
                          tokens=n, kv_heads=hkv)
            r["tokens_per_s"] = round(n / (r["us_median"] * 1e-6), 1)
            out["store_h%d_t%d" % (hkv, n)] = r
    return out


def tiny_decode_rows(torch, kvq):
    """The tiny decode (2 x 257 tokens, 8/2 heads, head_dim 64, unit scales):
    a latency row, the 514 tokens stored first."""
    from workloads import config_tiny_decode
    c = config_tiny_decode()
    dev = "cuda"
    cache = kvq.E4M3Cache(c.num_pages, c.num_kv_heads, c.head_dim)
    kvq.store(cache, c.k.to(dev), c.v.to(dev), torch.from_numpy(c.slot_mapping).to(dev), 1.0, 1.0)
    q = c.q.to(dev)
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device=dev)
    by = decode_bytes(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.max_seq_len)
    return {"tiny_decode": timed_row(torch, lambda i: kvq.decode(cache, q, bt, sl, c.max_seq_len, c.softmax_scale,
                                                                 1.0, 1.0, 1.0, out=out),
                                     "hbm", by, HBM_PEAK_GBPS, "GB/s", per=10, sha=case_sha(c),
                                     batch=c.batch, context=c.max_seq_len, note="latency-bound")}


def nvfp4_rows(torch, kvq):
    """NVFP4 368-byte records: bulk store of 524,288 tokens and MLA decode
    (batch 32 x 16,384 tokens, 16 heads). Algorithmic bytes: bf16 token in
    (1,152 B) + record out (368 B) + slot (8 B) per stored token; records +
    bf16 Q + bf16 O + block table + lengths per decode call."""
    from workloads import config_nvfp4_mla
    log("nvfp4 mla")
    c = config_nvfp4_mla(layer=0)
    sha = mla_sha(c)
    dev = "cuda"
    kv = c.kv.to(dev)
    slot = torch.from_numpy(c.slot_mapping).to(dev)
    caches = [kvq.Nvfp4Cache(c.num_pages) for _ in range(2)]
    T = int(kv.shape[0])
    sb = T * (576 * 2 + 368 + 8)
    rows = {}
    rows["nvfp4_store"] = timed_row(torch, lambda i: kvq.store(caches[i % 2], kv, None, slot, c.rope_scale),
                                    "hbm", sb, HBM_PEAK_GBPS, "GB/s", per=2, sha=sha, tokens=T)
    rows["nvfp4_store"]["tokens_per_s"] = round(T / (rows["nvfp4_store"]["us_median"] * 1e-6), 1)
    del kv
    q = c.q.to(dev)
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    out = torch.empty((c.batch, c.num_q_heads, 512), dtype=torch.bfloat16, device=dev)
    L = c.max_seq_len
    ws = torch.zeros(max(kvq.decode_workspace_bytes(caches[0], c.batch, L, 16), 1), dtype=torch.uint8, device=dev)
    by = c.batch * (L * 368 + c.num_q_heads * (576 + 512) * 2 + ((L + 15) // 16) * 4 + 4)
    # 2 x 241 MB of records alternate: more than the Infinity Cache
    rows["nvfp4_mla_decode"] = timed_row(
        torch, lambda i: kvq.decode(caches[i % 2], q, bt, sl, L, c.softmax_scale, k_scale=c.rope_scale, out=out,
                                    workspace=ws),
        "hbm", by, HBM_PEAK_GBPS, "GB/s", per=4, sha=sha, batch=c.batch, context=L, heads=c.num_q_heads,
        roof_extra={"kernels": "mla_decode_kernel + mla_combine_kernel"})
    del caches, q, out
    torch.cuda.empty_cache()
    rows.update(nvfp4_prefill_rows(torch, kvq))
    return rows


def nvfp4_prefill_rows(torch, kvq):
    """NVFP4 chunked prefill: 4 sequences x 16,384 tokens, the last 1,024 new,
    16 heads. Flops: 2 x (576 + 512) per attended (query row, head, key), the
    QK^T and PV multiply-adds; the kernel's MFMA runs in fp16."""
    from workloads import config_nvfp4_mla_prefill
    log("nvfp4 mla prefill")
    c = config_nvfp4_mla_prefill()
    sha = mla_sha(c)
    dev = "cuda"
    cache = kvq.Nvfp4Cache(c.num_pages)
    kvq.store(cache, c.kv.to(dev), None, torch.from_numpy(c.slot_mapping).to(dev), c.rope_scale)
    q = c.q.to(dev)
    cu = torch.from_numpy(c.cu_q_lens).to(dev)
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    out = torch.empty((q.shape[0], c.num_q_heads, 512), dtype=torch.bfloat16, device=dev)
    visits = 0
    for L, lq in zip(c.seq_lens, c.q_lens):
        visits += int(np.arange(L - lq + 1, L + 1, dtype=np.int64).sum())
    fl = 2 * (576 + 512) * c.num_q_heads * visits
    row = timed_row(torch, lambda i: kvq.prefill(cache, q, cu, int(c.q_lens.max()), bt, sl, c.max_seq_len,
                                                 c.softmax_scale, k_scale=c.rope_scale, out=out),
                    "mfma", fl, FP16_PEAK_TFLOPS, "TFLOP/s", per=1, sha=sha, batch=c.batch,
                    new_tokens=int(c.q_lens[0]), context=c.max_seq_len, roof_extra={"dtype": "fp16"})
    del cache
    torch.cuda.empty_cache()
    return {"nvfp4_mla_prefill": row}


def prefill_flops(seq_lens, q_lens, Hq, D, window=0):
    """QK^T and PV multiply-adds of causal chunked prefill, 2 flops each:
    4 * D per attended (query row, head, key). Nominal: every causal pair
    counts, also those whose probability is exactly zero under the bias,
    whose work the kernel skips."""
    visits = 0
    for L, lq in zip(seq_lens, q_lens):
        pos = np.arange(L - lq, L, dtype=np.int64)
        keys = pos + 1 if window <= 0 else np.minimum(pos + 1, window)
        visits += int(keys.sum())
    return 4 * D * Hq * visits


ISSUE_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "issue_counters.md")


def issue_record():
    """MfmaUtil / VALUBusy of the prefill kernels from the committed rocprofv3
    counter summary, or None when the kernel source changed since."""
    import hashlib
    try:
        line = [l for l in open(ISSUE_PROFILE) if l.startswith("issue_record: ")][0]
        rec = json.loads(line[len("issue_record: "):])
        h = hashlib.sha256(open(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                             rec["kernel_source"]), "rb").read()).hexdigest()
        return rec["kernels"] if h == rec["kernel_source_sha256"] else None
    except (OSError, IndexError, KeyError, ValueError):
        return None


def prefill_rows(torch, kvq):
    from workloads import config_chunked_prefill, rel_bias_table
    log("chunked prefill")
    c = config_chunked_prefill()
    sha = case_sha(c)
    dev = "cuda"
    k, v, q = c.k.to(dev), c.v.to(dev), c.q.to(dev)
    slot = torch.from_numpy(c.slot_mapping).to(dev)
    sc = {n: float(kvq.calibrate_amax(x)[1].item()) for n, x in (("k", k), ("v", v), ("q", q))}
    cache = kvq.E4M3Cache(c.num_pages, c.num_kv_heads, c.head_dim)
    cached, new = [torch.from_numpy(i).to(dev) for i in c.store_batches]
    kvq.store(cache, k[cached].contiguous(), v[cached].contiguous(), slot[cached], sc["k"], sc["v"])
    kn, vn, sn = k[new].contiguous(), v[new].contiguous(), slot[new].contiguous()
    T = int(kn.shape[0])
    rows = {}
    rows["store_prefill_new"] = timed_row(torch, lambda i: kvq.store(cache, kn, vn, sn, sc["k"], sc["v"]), "hbm",
                                          store_bytes(T, c.num_kv_heads, c.head_dim), HBM_PEAK_GBPS, "GB/s",
                                          per=10, sha=sha, tokens=T)
    del k, v
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    cu = torch.from_numpy(c.cu_q_lens).to(dev)
    slopes = torch.from_numpy(c.slopes).to(dev)
    out = torch.empty_like(q)
    fl = prefill_flops(c.seq_lens, c.q_lens, c.num_q_heads, c.head_dim)
    mix = {"dtype": "fp8 QK^T + fp16 PV", "peak_note": "half the flops at each MFMA rate"}
    issue = issue_record() or {}

    # the slope-bias calls' key-norm workspace, allocated once
    pws = torch.empty(max(kvq.prefill_workspace_bytes(cache, c.batch, c.max_seq_len, c.num_q_heads, slopes=slopes),
                          1), dtype=torch.uint8, device=dev)

    def run(**kw):
        if kw.get("slopes") is not None and kw.get("use_workspace", True):
            kw["workspace"] = pws
        return lambda i: kvq.prefill(cache, q, cu, c.max_q_len, bt, sl, c.max_seq_len, c.softmax_scale, sc["q"],
                                     sc["k"], sc["v"], out=out, **kw)
    shape = {"batch": c.batch, "new_tokens": int(c.q_lens[0]), "context": c.max_seq_len}
    # without a bias no probability underflows: every block is computed (the
    # kernel's dense rate)
    r = timed_row(torch, run(), "mfma", fl, PREFILL_MIXED_PEAK_TFLOPS, "TFLOP/s", per=1, sha=sha,
                  roof_extra=mix, **shape)
    r["pct_of_fp8_peak"] = round(100 * r["roofline"]["achieved"] / FP8_PEAK_TFLOPS, 2)
    if "prefill_e4m3_kernel<0, 0>" in issue:
        r.update(issue["prefill_e4m3_kernel<0, 0>"])
    rows["chunked_prefill_nobias"] = r
    # the slope bias (the workload's main row): blocks whose every probability
    # is exactly zero are skipped, so the flops are nominal
    r = timed_row(torch, run(slopes=slopes), "mfma", fl, PREFILL_MIXED_PEAK_TFLOPS, "TFLOP/s", per=1, sha=sha,
                  roof_extra=dict(mix, flops_kind="nominal: every causal pair, also skipped exact zeros; frac above 1 "
                                                    "means the skipped work outweighs the shortfall from peak"),
                  **shape)
    r["nominal_pct_of_fp8_peak"] = round(100 * r["roofline"]["achieved"] / FP8_PEAK_TFLOPS, 2)
    if "prefill_e4m3_kernel<1, 0>" in issue:
        r.update(issue["prefill_e4m3_kernel<1, 0>"])
    rows["chunked_prefill"] = r
    # the same call without the key-norm workspace: the early stop uses the
    # looser 448 * sum |q| bound (same output)
    r = timed_row(torch, run(slopes=slopes, use_workspace=False), "mfma", fl, PREFILL_MIXED_PEAK_TFLOPS, "TFLOP/s",
                  per=1, sha=sha, roof_extra=dict(mix, flops_kind="nominal"), **shape)
    rows["chunked_prefill_no_key_norms"] = r
    # the same prefill with a learned relative-bias table of 1,024 entries
    rel = torch.from_numpy(rel_bias_table(np.random.default_rng(6), c.num_q_heads, 1024)).to(torch.bfloat16).to(dev)
    r = timed_row(torch, run(rel_bias=rel), "mfma", fl, PREFILL_MIXED_PEAK_TFLOPS, "TFLOP/s", per=1, sha=sha,
                  roof_extra=mix, **shape)
    rows["chunked_prefill_rel1024"] = r
    # P variants on fp8 MFMA (slope bias): one e4m3 term (opt-in, looser
    # tolerance) and two e4m3 terms (the measured alternative to fp16 P)
    for name, kw in (("chunked_prefill_fp8p", {"fp8_p": True}), ("chunked_prefill_fp8p2", {"fp8_p2": True})):
        r = timed_row(torch, run(slopes=slopes, **kw), "mfma", fl, FP8_PEAK_TFLOPS, "TFLOP/s", per=1, sha=sha,
                      roof_extra={"dtype": "fp8", "flops_kind": "nominal"}, **shape)
        rows[name] = r
    del cache
    torch.cuda.empty_cache()
    return rows


def long_context_rows(torch, kvq):
    from workloads import config_long_context
    out = {}
    log("long-context decode")
    c = config_long_context()
    sha = case_sha(c)
    dev = "cuda"
    k, v, q = c.k.to(dev), c.v.to(dev), c.q.to(dev)
    slot = torch.from_numpy(c.slot_mapping).to(dev)
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    sc = {n: float(kvq.calibrate_amax(x)[1].item()) for n, x in (("k", k), ("v", v), ("q", q))}
    caches = [kvq.E4M3Cache(c.num_pages, c.num_kv_heads, c.head_dim) for _ in range(2)]
    for cache in caches:
        kvq.store(cache, k, v, slot, sc["k"], sc["v"])
    del k, v
    B, Hq, Hkv, D, L = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.max_seq_len
    outb = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    for w in (0, 512):
        ws = torch.zeros(max(kvq.decode_workspace_bytes(caches[0], B, L, Hq, window=w), 1), dtype=torch.uint8,
                         device=dev)
        att = min(L, w) if w else L
        by = decode_bytes(B, Hq, Hkv, D, att)
        out["long_context" + ("_window512" if w else "")] = timed_row(
            torch, lambda i, w=w, ws=ws: kvq.decode(caches[i % 2], q, bt, sl, L, c.softmax_scale, sc["q"], sc["k"],
                                                    sc["v"], window=w, out=outb, workspace=ws),
            "hbm", by, HBM_PEAK_GBPS, "GB/s", per=5, sha=sha, batch=B, context=L, attended=att,
            **({"note": "latency-bound"} if w else {}))
    del caches
    torch.cuda.empty_cache()
    return out


def mla_decode_only(torch, kvq):
    """The NVFP4 store and MLA decode rows without the prefill row (profiling)."""
    saved = globals()["nvfp4_prefill_rows"]
    globals()["nvfp4_prefill_rows"] = lambda torch, kvq: {}
    try:
        return nvfp4_rows(torch, kvq)
    finally:
        globals()["nvfp4_prefill_rows"] = saved


def tier1_rows(torch, kvq):
    """The two attention shapes of the vLLM PR 54705 evidence document ("Tier
    1: kernel performance") not covered by the workloads above:
    decode_kv65536_b1_tp4 (one sequence over 65,536 keys, 16/2 heads) and
    local_prefill_q8192_tp1 (8,192 new tokens, window 512, 64/8 heads, learned
    bias of extent 128)."""
    from workloads import config_single_stream_decode, config_local_prefill
    log("tier-1 shapes")
    dev = "cuda"
    rows = {}
    c = config_single_stream_decode()
    sha = case_sha(c)
    k, v, q = c.k.to(dev), c.v.to(dev), c.q.to(dev)
    slot = torch.from_numpy(c.slot_mapping).to(dev)
    sc = {n: float(kvq.calibrate_amax(x)[1].item()) for n, x in (("k", k), ("v", v), ("q", q))}
    # 10 copies of the 33.5 MB cache rotate, 335 MB: more than the Infinity Cache
    caches = [kvq.E4M3Cache(c.num_pages, c.num_kv_heads, c.head_dim) for _ in range(10)]
    for cache in caches:
        kvq.store(cache, k, v, slot, sc["k"], sc["v"])
    del k, v
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    L, Hq, Hkv, D = c.max_seq_len, c.num_q_heads, c.num_kv_heads, c.head_dim
    outb = torch.empty((1, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(kvq.decode_workspace_bytes(caches[0], 1, L, Hq), 1), dtype=torch.uint8, device=dev)
    rows["single_stream_decode"] = timed_row(
        torch, lambda i: kvq.decode(caches[i % 10], q, bt, sl, L, c.softmax_scale, sc["q"], sc["k"], sc["v"],
                                    out=outb, workspace=ws),
        "hbm", decode_bytes(1, Hq, Hkv, D, L), HBM_PEAK_GBPS, "GB/s", per=10, sha=sha, batch=1, context=L,
        q_heads=Hq, kv_heads=Hkv)
    del caches
    torch.cuda.empty_cache()
    c = config_local_prefill()
    sha = case_sha(c)
    k, v, q = c.k.to(dev), c.v.to(dev), c.q.to(dev)
    slot = torch.from_numpy(c.slot_mapping).to(dev)
    sc = {n: float(kvq.calibrate_amax(x)[1].item()) for n, x in (("k", k), ("v", v), ("q", q))}
    cache = kvq.E4M3Cache(c.num_pages, c.num_kv_heads, c.head_dim)
    kvq.store(cache, k, v, slot, sc["k"], sc["v"])
    del k, v
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seq_lens).to(dev)
    cu = torch.from_numpy(c.cu_q_lens).to(dev)
    rel = torch.from_numpy(c.rel).to(torch.bfloat16).to(dev)
    out = torch.empty_like(q)
    fl = prefill_flops(c.seq_lens, c.q_lens, c.num_q_heads, c.head_dim, window=c.window)
    rows["local_prefill"] = timed_row(
        torch, lambda i: kvq.prefill(cache, q, cu, c.max_q_len, bt, sl, c.max_seq_len, c.softmax_scale, sc["q"],
                                     sc["k"], sc["v"], window=c.window, rel_bias=rel, out=out),
        "mfma", fl, PREFILL_MIXED_PEAK_TFLOPS, "TFLOP/s", per=2, sha=sha,
        roof_extra={"dtype": "fp8 QK^T + fp16 PV"}, new_tokens=int(c.q_lens[0]), window=c.window,
        q_heads=c.num_q_heads, kv_heads=c.num_kv_heads, rel_extent=int(c.rel.shape[1]))
    del cache
    torch.cuda.empty_cache()
    return rows


def cpu_baseline(c):
    """The oracle, as it stands, on a bounded sample of the same workload:
    decode attention (page gather, Q quantization, fp64 attention) for 64
    sequences, and quant-on-store of 2 sequences' tokens."""
    from threadpoolctl import threadpool_info
    from oracle.kvcache import new_cache, store_e4m3, calibrate_amax
    from oracle.attention import paged_decode
    log("cpu oracle baseline")
    k = c.k.float().numpy()
    v = c.v.float().numpy()
    q = c.q.float().numpy()
    _, sk = calibrate_amax(k)
    _, sq = calibrate_amax(q)
    sv = c.v_scale_override
    L = c.max_seq_len
    n_store = 2
    tok = np.arange(n_store * L)
    kc, vc = new_cache(c.num_pages, c.num_kv_heads, 16, c.head_dim)
    t0 = time.perf_counter()
    store_e4m3(kc, vc, k[tok], v[tok], c.slot_mapping[tok], sk, sv)
    t_store = time.perf_counter() - t0
    # decode: reuse the stored pages of the first sequences for every sampled
    # sequence (same shapes and work per sequence)
    bt = c.block_table.copy()
    for b in range(c.batch):
        bt[b] = c.block_table[b % n_store]
    t0 = time.perf_counter()
    paged_decode(q, kc, vc, bt, c.seq_lens, c.softmax_scale, sq, sk, sv)
    t_dec = time.perf_counter() - t0
    by = decode_bytes(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, L)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(by / t_dec / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "decode attention of all 64 sequences x 8,192 tokens (%.1f s) and "
                      "quant-on-store of %d sequences (%d tokens, %.1f s) of the batched-decode "
                      "workload; numpy fp64" % (t_dec, n_store, len(tok), t_store),
            "store_tokens_per_s": round(len(tok) / t_store, 1),
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
