// Internal launch interface between the C-ABI layer (kvq_api.hip) and the
// kernel translation units. Host code only; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

struct StoreE4M3Launch {
  const uint16_t *k, *v;
  int64_t k_stride, v_stride;  // elements between tokens
  const int64_t *slot;
  int64_t num_tokens;
  uint8_t *kc, *vc;
  int hkv, d;
  float k_inv, v_inv;          // fp32(1/scale), computed on the host
};
hipError_t launch_store_e4m3(const StoreE4M3Launch &a, hipStream_t s);

struct StoreNvfp4Launch {
  const uint16_t *x;           // [T][576] bf16
  int64_t stride;
  const int64_t *slot;
  int64_t num_tokens;
  uint8_t *records;            // [pages][16][368]
  float rope_inv;              // fp32(1/rope_scale)
  float static_s2;             // 0: per-token s2 = amax / 2688; > 0: this outer scale for every token
};
hipError_t launch_store_nvfp4(const StoreNvfp4Launch &a, hipStream_t s);

struct AmaxLaunch {
  const uint16_t *x;
  int64_t rows, row_len, row_stride;
  const int64_t *slot;
  float *amax_inout;
  float *scale_out;
};
hipError_t launch_amax(const AmaxLaunch &a, int num_cus, hipStream_t s);
hipError_t launch_scale_rule(const float *amax, int rule, float *scale, hipStream_t s);

struct BandLaunch {
  const uint16_t *x;
  int64_t rows, row_len, row_stride;
  const int64_t *slot;
  float inv;                   // fp32(1/scale), computed on the host as the store does
  unsigned long long *counts;  // [2]: clipped, flushed
};
hipError_t launch_band_counts(const BandLaunch &a, int num_cus, hipStream_t s);

// Split plan of the e4m3 decode kernel.
struct DecodePlan {
  int waves;        // waves per workgroup (1, 2, 4 or 8)
  int splits;       // KV splits per (sequence, KV head, query tile)
  int blocks_per_split;  // 128-key blocks (8 pages) per split
  int qtiles;       // ceil(group / 16)
  size_t workspace; // bytes of partials (0 when splits == 1)
};

struct DecodeE4M3Launch {
  const uint16_t *q;           // [B][Hq][D]
  const uint8_t *kc, *vc;
  const int32_t *block_table;
  int64_t bt_stride;
  const int32_t *seq_lens;
  const float *slopes;         // [Hq] or nullptr
  const uint16_t *rel;         // bf16 [Hq][rel_extent] or nullptr
  int rel_extent;
  uint16_t *out;               // [B][Hq][D]
  float *part_o;               // [B][Hq][S][D]
  float *part_ml;              // [B][Hq][S][2]
  int batch, hq, hkv, d, window;
  float q_inv;                 // fp32(1/q_scale)
  float fold_log2;             // softmax_scale * q_scale * k_scale * log2(e)
  float v_scale;
  // fused append (nullptr: none): the current token's bf16 K/V [B][Hkv][D],
  // quantized with k_inv / v_inv and written at position seq_lens[b] - 1
  const uint16_t *k_new, *v_new;
  uint8_t *kc_w, *vc_w;        // the same pools as kc / vc, writable
  float k_inv, v_inv;
};
hipError_t launch_decode_e4m3(const DecodeE4M3Launch &a, const DecodePlan &p, hipStream_t s);

struct PrefillE4M3Launch {
  const uint16_t *q;           // [total_q][Hq][D]
  const int32_t *cu_q_lens;
  const uint8_t *kc, *vc;
  const int32_t *block_table;
  int64_t bt_stride;
  const int32_t *seq_lens;
  const float *slopes;         // [Hq] or nullptr
  const uint16_t *rel;         // bf16 [Hq][rel_extent] or nullptr
  int rel_extent;
  uint16_t *out;
  int batch, hq, hkv, d, window, max_q_len;
  int p_mode;                  // P of PV: 0 fp16; 1 one e4m3 term, 2 two e4m3 terms (both
                               // with a lazy rescale of slack 0.75, on fp8 MFMA)
  float q_inv, fold_log2, v_scale;
  // slope bias only (nullptr: not used): per (sequence, KV head, 128-key
  // block) the largest Euclidean norm of the block's key codes,
  // [batch][hkv][knorm_blocks], written by a launch before the prefill's
  int knorm_blocks;
  float *knorm;
};
hipError_t launch_prefill_e4m3(const PrefillE4M3Launch &a, hipStream_t s);

struct DecodeMlaLaunch {
  const uint16_t *q;           // [B][Hq][576]
  const uint8_t *records;
  const int32_t *block_table;
  int64_t bt_stride;
  const int32_t *seq_lens;
  uint16_t *out;               // [B][Hq][512]
  float *part_o;               // [B][Hq][S][512]
  float *part_ml;              // [B][Hq][S][4]: M, den, E, pad
  int batch, hq;
  float scale_log2;            // softmax_scale * log2(e)
  float rope_scale;
  // prefill (extend) mode when cu_q_lens is set: q / out rows
  // cu_q_lens[b] .. cu_q_lens[b+1]-1, one workgroup per row, one split
  const int32_t *cu_q_lens;
  int max_q_len;
};
hipError_t launch_prefill_mla(const DecodeMlaLaunch &a, int max_seq_len, hipStream_t s);
struct MlaPlan {
  int splits;
  int pages_per_split;
  size_t workspace;
};
hipError_t launch_decode_mla(const DecodeMlaLaunch &a, const MlaPlan &p, hipStream_t s);

// Decode entry shared by the public decode calls (kvq_api.hip). decode_check
// runs every host-side check of the arguments except the workspace and sets
// the workspace bytes the call needs (0 when num_seqs is 0 or one split
// suffices); decode_run checks again, checks the workspace and launches.
// k_new / v_new non-null: the fused append.
int decode_check(const kvq_cache *cache, const void *q, const void *k_new, const void *v_new,
                 const int32_t *block_table, int64_t block_table_stride, const int32_t *seq_lens,
                 int32_t num_seqs, int32_t max_seq_len, const kvq_attn_params *params, void *out,
                 size_t *workspace_needed);
int decode_run(const kvq_cache *cache, const void *q, const void *k_new, const void *v_new,
               const int32_t *block_table, int64_t block_table_stride, const int32_t *seq_lens,
               int32_t num_seqs, int32_t max_seq_len, const kvq_attn_params *params, void *out,
               void *workspace, size_t workspace_bytes, kvq_stream_t stream);

}  // namespace kvq
