/*
 * kvq: quantized-KV-cache attention for AMD MI355X (gfx950).
 *
 * C ABI of libkvq.so. Plain pointers and sizes only. Device pointers point to
 * HIP device memory owned by the caller; the library allocates nothing,
 * copies nothing between host and device and never synchronizes: every call
 * enqueues its kernels on the given stream and returns. Pointers must stay
 * valid until that stream work completes.
 *
 * Sources of the operations (pages cited by title and section):
 *  [PR54705] vLLM PR 54705, "opt-in fp8 e4m3 KV cache for the Inkling model on
 *            SM100": section "Purpose" (gate, query quantization, quant-on-store
 *            with a clamp to the e4m3 finite range, descale handling, cache
 *            plumbing) and the evidence document ("Tier 0" online softmax and
 *            fp8 P, "Tier 1" write path, "Tier 2" stored-value statistics).
 *  [KVcal]   Qwen3.8-27B-FP8-KVcal model card: scale table (amax/448) and
 *            "Rebuild / reproduce" (running amax).
 *  [PR189]   local-inference-lab/vllm PR 189, "mla: wire dynamic per-token
 *            NVFP4 scaling and cache ABI": commit message, "Why", "Changes".
 *
 * Error behaviour. Every entry point validates its host-visible arguments
 * before enqueueing anything and returns a kvq_status; nothing is launched
 * when the status is not KVQ_OK. Device-resident contents (block-table
 * entries, slot values, sequence lengths) are trusted: the caller guarantees
 * that block-table entries for pages a sequence uses are < num_pages, that
 * slots are < num_pages * page_size and unique within one store call, and
 * that every seq_lens[b] <= max_seq_len.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 7

/* A hipStream_t. NULL selects the null stream. */
typedef struct ihipStream_t *kvq_stream_t;

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* NULL pointer, bad size, stride or alignment */
  KVQ_ERR_UNSUPPORTED = -2, /* format/shape this library does not implement:
                               unknown cache formats (e5m2, FNUZ e4m3 ...) fail
                               here instead of running with wrong numerics,
                               [PR54705] "Purpose", gate bullet */
  KVQ_ERR_BAD_SCALE = -3,   /* a scale that is not finite and > 0,
                               [PR54705] "Purpose", unity-scale bullet */
  KVQ_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required */
  KVQ_ERR_HIP = -5,         /* a HIP runtime call or launch failed */
  KVQ_ERR_SCRATCH_LIMIT = -6 /* kvq_paged_attn_decode_noalloc: the call's split
                               partials exceed the library's static scratch
                               array (KVQ_NOALLOC_SCRATCH_BYTES) */
} kvq_status;

typedef enum {
  /* OCP e4m3fn (max 448) with one fp32 scale per tensor ([PR54705]). */
  KVQ_FMT_E4M3 = 1,
  /* 368-byte NVFP4 latent record with a per-token outer scale ([PR189]). */
  KVQ_FMT_NVFP4_MLA368 = 2
} kvq_format;

/*
 * Paged cache descriptor (caller-owned device memory, raw bytes; the pages'
 * pool is uint8 viewed as e4m3, [PR54705] "Purpose", cache-plumbing bullet).
 * slot = page * page_size + offset.
 *
 * KVQ_FMT_E4M3:
 *   k : u8 [num_pages][num_kv_heads][page_size][head_dim]   (token rows)
 *   v : u8 [num_pages][num_kv_heads][head_dim][page_size]   (token-minor:
 *       the 16 tokens of one dim are contiguous, the layout PV consumes)
 *   head_dim 64 or 128; page_size 16; both pointers 16-byte aligned.
 * KVQ_FMT_NVFP4_MLA368:
 *   k : u8 [num_pages][page_size][368] records; v must be NULL;
 *   num_kv_heads 1, head_dim 576 (512 latent + 64 RoPE), page_size 16.
 *   Record: [0,256) e2m1 values, element 2i in the low nibble of byte i;
 *   [256,288) 32 E4M3 group scales (16 elements per group); [288,292) zero;
 *   [292,296) per-token fp32 outer scale, little endian ([PR189] commit
 *   message: the scale sits at [292,296) of existing padding); [296,304)
 *   zero; [304,368) 64 e4m3 RoPE codes.
 */
typedef struct {
  int32_t format;       /* kvq_format */
  int32_t page_size;    /* tokens per page; must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t num_pages;
  void *k;
  void *v;
} kvq_cache;

/*
 * Attention parameters, passed by value-struct pointer (host memory). Scales
 * are host floats: the hot path never reads a scale back from the GPU
 * ([PR54705] "Purpose", query-quantization bullet).
 */
typedef struct {
  int32_t num_q_heads;   /* multiple of num_kv_heads; query head h reads KV
                            head h / (num_q_heads / num_kv_heads) */
  int32_t window;        /* 0: full attention; W > 0: a query at position p
                            attends keys j with p - W < j <= p (a 512-token
                            window is [PR54705] "Purpose") */
  int32_t num_splits;    /* 0: library's choice; > 0 requests the number of
                            KV splits per (sequence, KV head) in decode. The
                            library clamps it: e4m3, at least one 128-key
                            block (8 pages) per split; NVFP4, at least 4 and
                            at most 512 pages per split */
  int32_t rel_extent;    /* entries per head of rel_bias, 1 .. 1,048,576,
                            when rel_bias is set; 0 otherwise */
  float softmax_scale;   /* finite, > 0 */
  float q_scale;         /* E4M3: Q quantization scale; NVFP4: ignored */
  float k_scale;         /* E4M3: K descale; NVFP4: RoPE descale */
  float v_scale;         /* E4M3: V descale; NVFP4: ignored */
  const float *alibi_slopes; /* device fp32 [num_q_heads] or NULL: additive
                            bias bf16(slope_h * -(p - j)) added after the
                            descaled QK^T, [PR54705] "Purpose", descale bullet */
  const uint16_t *rel_bias; /* device bf16 [num_q_heads][rel_extent] or NULL:
                            learned relative bias ([PR54705] "Environment":
                            the model's learned relative position bias;
                            "Test Plan": extents 128 and 1024),
                            bias(h, p, j) = rel_bias[h][min(p - j, rel_extent - 1)]
                            added where the slope bias is. At most one of
                            alibi_slopes and rel_bias may be set. */
  uint32_t flags;        /* KVQ_FLAG_* bits; other bits must be 0 */
} kvq_attn_params;

/* kvq_attn_params.flags */
enum {
  /* Prefill only (decode ignores it): P = 2^8 p as a single e4m3 term with a
     lazily raised running max (slack 0.75 in log2 units, under the
     log2(448) - 8 = 0.807 bound) and PV on fp8 MFMA ([PR54705] evidence
     "Tier 0"). A speed variant: its error is within the pages' fp8 test
     tolerance (atol and rtol 0.15, [PR54705] "Test Plan"), not within this
     library's default attention tolerance, so it is off unless requested. */
  KVQ_FLAG_PREFILL_FP8_P = 1u,
  /* Prefill only: P = 2^8 p as two e4m3 terms (hi = e4m3(P), lo = e4m3(P -
     hi)) on fp8 MFMA, with the same lazy running max (slack 0.75) and a
     normaliser summed from the same two terms ([PR54705] evidence "Tier 0"
     for the 2^8 pre-scale and its log2(448) - 8 bound). About 8 significant
     bits per weight (the default fp16 P keeps 11); the fp8-PV path, within
     the default tolerance, kept beside the default for its measured
     comparison: blocks whose every P rounds to zero are skipped, and e4m3
     P = 2^(x - m + 8) reaches zero 19 log2 units below the running max
     against 26 for fp16 P, so with a decaying bias this path skips more and
     can be the faster one; without a bias it is the slower one (two fp8
     MFMAs cost what one fp16 MFMA does, and the split costs vector
     instructions). At most one of the two flags may be set. */
  KVQ_FLAG_PREFILL_FP8_P2 = 2u
};

/*
 * kvq_store: quant-on-store ([PR54705] "Purpose", quant-on-store bullet;
 * "Tier 1" write path: multiply + clamp + convert).
 *
 * KVQ_FMT_E4M3: k, v are bf16 [num_tokens][num_kv_heads][head_dim] with
 *   k_token_stride / v_token_stride elements between tokens (heads and dims
 *   contiguous). Each element becomes e4m3_RNE(clamp(x * fp32(1/scale),
 *   -448, 448)) (NaN stays NaN) and is written at slot_mapping[t]; tokens
 *   with slot < 0 are skipped. Strides must be multiples of 8 elements and
 *   k, v 16-byte aligned.
 * KVQ_FMT_NVFP4_MLA368: k is bf16 [num_tokens][576] (latent then RoPE) with
 *   k_token_stride; v must be NULL; k_scale is the RoPE scale; v_scale is
 *   ignored. Writes one 368-byte record per token: s2 = amax(latent)/2688,
 *   per 16-element group sg = e4m3(min(ag / (6 s2), 448)), values
 *   e2m1(clip(x / (e4m3(sg) s2), -6, 6)) ([PR189] "Why": the outer scale is
 *   derived per token and stored in the record).
 * num_tokens == 0 returns KVQ_OK without launching.
 */
int kvq_store(const kvq_cache *cache, const void *k, int64_t k_token_stride,
              const void *v, int64_t v_token_stride, const int64_t *slot_mapping,
              int64_t num_tokens, float k_scale, float v_scale, kvq_stream_t stream);

/*
 * kvq_store_nvfp4_static: the NVFP4 record store with one static outer scale
 * for every token instead of the per-token one ([PR189] commit message: the
 * writer's outer scale was statically 1.0, or calibrated per layer by a
 * separate static mode; "Why": with it, low-magnitude layers put many group
 * scales into e4m3's subnormal range). It exists for the A/B against the
 * per-token scale.
 *
 * cache must be KVQ_FMT_NVFP4_MLA368 (else KVQ_ERR_UNSUPPORTED). x, token_stride,
 * slot_mapping, num_tokens and rope_scale as for kvq_store. outer_scale
 * (finite, > 0, else KVQ_ERR_BAD_SCALE) replaces amax(latent)/2688 as s2 in
 * every formula of kvq_store and is written to bytes [292, 296), so the
 * readers of this library decode static and per-token records alike. The
 * pages' static records carry no scale in the record and take it at launch;
 * the arithmetic is the same.
 */
int kvq_store_nvfp4_static(const kvq_cache *cache, const void *x, int64_t token_stride,
                           const int64_t *slot_mapping, int64_t num_tokens, float rope_scale,
                           float outer_scale, kvq_stream_t stream);

/*
 * kvq_calibrate_amax: running amax and scale = amax / 448 ([KVcal] scale
 * table; "Rebuild / reproduce": running |K|/|V| amax over calls; [PR54705]
 * "Tier 2": only the values actually stored).
 *
 * x: bf16 [num_rows][row_len] with row_stride elements between rows
 * (row_len and row_stride multiples of 8, x 16-byte aligned). Rows whose
 * slot_mapping entry is < 0 are ignored (slot_mapping may be NULL: all rows).
 * amax_inout: device fp32, must hold a value >= 0 (0 to start); it becomes
 * max(amax_inout, max |x|). scale_out: device fp32 or NULL; receives
 * fp32(amax_inout / 448) after the update. The result is bit-exact and
 * independent of launch order (integer max of |bf16| bit patterns).
 * num_rows == 0 still writes scale_out from the unchanged amax.
 */
int kvq_calibrate_amax(const void *x, int64_t num_rows, int64_t row_len,
                       int64_t row_stride, const int64_t *slot_mapping,
                       float *amax_inout, float *scale_out, kvq_stream_t stream);

/* Scale rules of kvq_scale_from_amax. */
enum kvq_scale_rule {
  KVQ_SCALE_AMAX_448 = 0,   /* fp32(amax) / fp32(448) ([KVcal] scale table) */
  KVQ_SCALE_CEIL_BF16 = 1,  /* the smallest bf16 >= fp32(amax) / fp32(448),
                               stored as fp32 ([KVcal] "Rebuild / reproduce":
                               ceil_to_bfloat16) */
  KVQ_SCALE_SAFETY_1P3 = 2  /* max(1, amax * 1.3 / 448) in fp64, rounded to
                               fp32 ([PR54705] evidence "Tier 4": the
                               calibration utility's rule) */
};

/*
 * kvq_scale_from_amax: *scale_out = rule(*amax), computed on the device (no
 * read-back). amax: device fp32, e.g. the running amax of
 * kvq_calibrate_amax; scale_out: device fp32. NULL pointers or an unknown
 * rule: KVQ_ERR_INVALID_ARG. Bit-exact: one fp32 division for the first two
 * rules, fp64 multiply and divide for the third.
 */
int kvq_scale_from_amax(const float *amax, int32_t rule, float *scale_out, kvq_stream_t stream);

/*
 * kvq_band_counts: exact e4m3 band counters of the values a store at `scale`
 * would write ([PR54705] evidence "Tier 2": clip and flush-to-zero counts of
 * the stored values at a given scale). x, num_rows, row_len, row_stride and
 * slot_mapping as in kvq_calibrate_amax. With y = fp32(x) * fp32(1/scale)
 * (the store's arithmetic):
 *   counts_inout[0] += values with |y| > 448, which the clamp changes
 *                      (infinities counted, NaN not);
 *   counts_inout[1] += nonzero values whose e4m3 code is +0 or -0 (NaN not).
 * counts_inout: device uint64 [2], 8-byte aligned, accumulated across calls
 * (the caller zeroes it to start). scale must be finite and > 0
 * (KVQ_ERR_BAD_SCALE). Exact integer counts, independent of launch order.
 * num_rows == 0 returns KVQ_OK without launching.
 */
int kvq_band_counts(const void *x, int64_t num_rows, int64_t row_len, int64_t row_stride,
                    const int64_t *slot_mapping, float scale, uint64_t *counts_inout,
                    kvq_stream_t stream);

/*
 * Workspace (device bytes) kvq_paged_attn_decode needs for these arguments
 * on the current device. 0 means no workspace is needed. Returns 0 for
 * invalid arguments as well (the decode call reports those).
 */
size_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t num_seqs,
                                  int32_t max_seq_len, const kvq_attn_params *params);

/*
 * kvq_paged_attn_decode: one new query token per sequence, at position
 * seq_lens[b] - 1 (the current token's K/V must already be stored).
 *
 * KVQ_FMT_E4M3 ([PR54705] "Purpose"): q bf16 [num_seqs][num_q_heads][head_dim]
 *   contiguous, 16-byte aligned. Q is quantized with the store's quantizer and
 *   q_scale; s = (Q8 . K8) * (softmax_scale * q_scale * k_scale) + bias;
 *   softmax over the attended keys; out = v_scale * sum_j p_j V8_j.
 * KVQ_FMT_NVFP4_MLA368 ([PR189]): q bf16 [num_seqs][num_q_heads][576], not
 *   quantized; K = [latent ; RoPE] decoded from the records (latent =
 *   e2m1 * group scale * record outer scale, RoPE = e4m3 * k_scale), V =
 *   latent; out bf16 [num_seqs][num_q_heads][512]. num_q_heads must be 16,
 *   max_seq_len at most 524,288, window 0 and both biases NULL
 *   (KVQ_ERR_UNSUPPORTED otherwise).
 *
 * block_table: device int32 [num_seqs][block_table_stride], pages of each
 * sequence in order. seq_lens: device int32 [num_seqs]. max_seq_len: a host
 * upper bound of seq_lens (no device read-back). out: bf16
 * [num_seqs][num_q_heads][head_dim_v]. A sequence of length 0 outputs zeros.
 * workspace: device memory of at least kvq_decode_workspace_bytes(...)
 * bytes (may be NULL when that is 0). num_seqs == 0 returns KVQ_OK.
 */
int kvq_paged_attn_decode(const kvq_cache *cache, const void *q,
                          const int32_t *block_table, int64_t block_table_stride,
                          const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len,
                          const kvq_attn_params *params, void *out, void *workspace,
                          size_t workspace_bytes, kvq_stream_t stream);

/*
 * kvq_paged_attn_decode_append: kvq_store of each sequence's current token
 * followed by kvq_paged_attn_decode, in one launch ([PR54705] "Purpose":
 * quant-on-store of K/V, then decode with the descale fold). KVQ_FMT_E4M3
 * only (KVQ_ERR_UNSUPPORTED otherwise).
 *
 * k_new, v_new: device bf16 [num_seqs][num_kv_heads][head_dim], contiguous,
 * 16-byte aligned: the K/V of the token at position seq_lens[b] - 1. They are
 * quantized exactly as kvq_store does with params->k_scale / v_scale and
 * written into the page the block table gives for that position; then the
 * attention reads them like every other stored token. The stored bytes and
 * the output equal those of kvq_store (at the same slots) followed by
 * kvq_paged_attn_decode. Sequences of length 0 store nothing. All other
 * arguments, the workspace and the errors are those of
 * kvq_paged_attn_decode (kvq_decode_workspace_bytes applies unchanged).
 */
int kvq_paged_attn_decode_append(const kvq_cache *cache, const void *q, const void *k_new,
                                 const void *v_new, const int32_t *block_table,
                                 int64_t block_table_stride, const int32_t *seq_lens,
                                 int32_t num_seqs, int32_t max_seq_len,
                                 const kvq_attn_params *params, void *out, void *workspace,
                                 size_t workspace_bytes, kvq_stream_t stream);

/*
 * kvq_paged_attn_decode_noalloc: kvq_paged_attn_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). It takes no workspace: the split
 * partials go to a static device array of the library,
 * KVQ_NOALLOC_SCRATCH_BYTES per device, which each device holds from this
 * entry point's first call on it until the process ends. The call allocates
 * nothing; its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress), with that device current.
 *
 * Arguments, arithmetic, output and errors are those of kvq_paged_attn_decode
 * (same kernels, same split plan: the output is bit-identical), plus
 * KVQ_ERR_SCRATCH_LIMIT, returned before anything is launched, when
 * kvq_decode_workspace_bytes(...) for these arguments exceeds
 * KVQ_NOALLOC_SCRATCH_BYTES (lower num_splits, or use kvq_paged_attn_decode
 * with a workspace). Every call on one device shares its array and leaves the
 * last call's partials in it (nothing there needs to start at zero: each
 * partial is written before it is read within the call): two calls that
 * overlap in time on one device (different streams, no ordering between
 * them) race and may return wrong outputs. Calls ordered on one stream are
 * safe.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int kvq_paged_attn_decode_noalloc(const kvq_cache *cache, const void *q,
                                  const int32_t *block_table, int64_t block_table_stride,
                                  const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                  const kvq_attn_params *params, void *out, kvq_stream_t stream);

/*
 * kvq_paged_attn_prefill: chunked prefill over the e4m3 cache ([PR54705]
 * "Purpose"; evidence "Tier 1" chunked-prefill case), or over NVFP4 records
 * ([PR189] "Changes" and "Validation": the readers apply the per-token outer
 * scale in decode and in prefill).
 *
 * The new queries of sequence b are rows cu_q_lens[b] .. cu_q_lens[b+1]-1 of
 * q bf16 [total_q][num_q_heads][head_dim] (contiguous, 16-byte aligned); query
 * i of the sequence sits at position seq_lens[b] - q_len_b + i (the new
 * tokens' K/V must already be stored) and attends keys j <= its position
 * (and > position - window when window > 0). Scores, bias and output as in
 * decode. cu_q_lens: device int32 [num_seqs + 1]; max_q_len: host upper
 * bound of the per-sequence query counts. out: bf16 [total_q][num_q_heads]
 * [head_dim_v]. KVQ_FMT_E4M3 needs head_dim 128. KVQ_FMT_NVFP4_MLA368: q is
 * bf16 [total_q][16][576] (not quantized), out bf16 [total_q][16][512], the
 * arithmetic of the NVFP4 decode; num_q_heads must be 16, max_seq_len at
 * most 32,768, window 0 and both biases NULL (KVQ_ERR_UNSUPPORTED
 * otherwise).
 *
 * workspace (optional): with the e4m3 cache and per-head slopes, a workspace
 * of at least kvq_prefill_workspace_bytes(...) bytes (4-byte aligned) lets
 * the call first compute, for every (sequence, KV head, 128-key block), the
 * largest Euclidean norm of the block's stored key codes (one extra launch
 * reading the attended K bytes once). A tile then leaves its key walk as soon
 * as |q . k| <= |q| |k| (Cauchy-Schwarz, over the codes) plus the bias at the
 * nearest remaining distance puts every remaining score at least the zero cut
 * below the running max, i.e. where every remaining probability rounds to
 * exactly zero. Without it (NULL, or fewer bytes) the walk uses the looser
 * bound 448 * sum |q|. The output is bit-identical either way; the workspace
 * holds nothing the caller needs afterwards. Other cases need no workspace
 * (workspace may be NULL, workspace_bytes 0).
 */
int kvq_paged_attn_prefill(const kvq_cache *cache, const void *q, const int32_t *cu_q_lens,
                           int64_t total_q, int32_t max_q_len, const int32_t *block_table,
                           int64_t block_table_stride, const int32_t *seq_lens,
                           int32_t num_seqs, int32_t max_seq_len,
                           const kvq_attn_params *params, void *out, void *workspace,
                           size_t workspace_bytes, kvq_stream_t stream);

/*
 * Workspace (device bytes) that lets kvq_paged_attn_prefill bound the
 * remaining scores by the per-block key norms: with the e4m3 cache and
 * per-head slopes, 4 * num_seqs * num_kv_heads * ceil(max_seq_len / 128);
 * 0 otherwise (and for invalid arguments, which the prefill call reports).
 */
size_t kvq_prefill_workspace_bytes(const kvq_cache *cache, int32_t num_seqs,
                                   int32_t max_seq_len, const kvq_attn_params *params);

/* Static text for a kvq_status value. */
const char *kvq_status_str(int status);

/* KVQ_ABI_VERSION of the loaded library. */
int kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
