"""Seeded synthetic inputs for the quantized-KV-cache attention path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
bench. It draws random numbers, rounds them to bf16 (the dtype the attention
layer hands to the cache) and lays tokens out in pages. It holds none of the
method's arithmetic: no quantisation, no scale rule, no attention.

Workload shapes and value distributions stand in for the pages' measurements:
  * e4m3 K/V/Q cache: the 16-token pages, 512-token sliding window and V
    outliers reaching 1,272 of the vLLM PR 54705 evidence document
    ("Tier 2: KV value range at unity scale"), and post-norm K/Q amax of
    about 20 from the Qwen3.8-27B-FP8-KVcal model card ("Observation point");
  * NVFP4 MLA latents: per-layer magnitude spread from small to large, the
    regime that motivates the per-token outer scale in local-inference-lab/vllm
    PR 189 ("Why").
"""
from .gen import (  # noqa: F401
    AttnCase,
    MlaCase,
    bf16,
    paged_layout,
    rel_bias_table,
    make_attn_case,
    make_mla_case,
    config_tiny_decode,
    config_batched_decode,
    config_long_context,
    config_chunked_prefill,
    config_single_stream_decode,
    config_local_prefill,
    write_path_tokens,
    config_nvfp4_mla,
    config_nvfp4_mla_prefill,
    geometric_slopes,
    CONFIGS,
)
