"""CPU oracle for the quantized-KV-cache attention path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
reference written in numpy (fp64 for attention, exact fp32 emulation wherever
the method fixes fp32 arithmetic). Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it. It shares no code with
the HIP library: not a kernel, header, table or constant generator.

Sources (cited by page title and section):
  * vLLM PR 54705, "opt-in fp8 e4m3 KV cache for the Inkling model on SM100":
    "Purpose" (quant-on-store with a clamp to the e4m3 finite range, static
    per-tensor Q quantisation, QK descale folded into the softmax scale ahead
    of an exact bf16 relative bias, V descale applied to the output), and the
    evidence document's "Tier 0" (fp8 P pre-scaled by 2^8 inside online
    softmax), "Tier 1" (multiply + clamp + convert on store) and "Tier 2"
    (statistics over exactly the stored values; exact e4m3 clip and
    flush-to-zero band counters), "Tier 4" (the safety-1.3 scale rule), and
    "Environment" / "Test Plan" (a learned relative position bias, extents
    128 and 1024).
  * Qwen3.8-27B-FP8-KVcal model card: the scale table (amax/448 for k, v and q;
    prob scale 1/448) and "Rebuild / reproduce" (running amax over calls;
    the ceil_to_bfloat16 scale rule).
  * local-inference-lab/vllm PR 189, "mla: wire dynamic per-token NVFP4 scaling
    and cache ABI": commit message and "Why" (368-byte record, e2m1 values with
    E4M3 group scales, a per-token fp32 outer scale at record bytes [292,296),
    FP8 RoPE part).

Parity status per function is listed in each module's header.
"""
from . import codecs, kvcache, attention, nvfp4, calibration  # noqa: F401
