// C ABI of libkvq.so: argument validation, split planning and launches.
// Every check here runs on the host before anything is enqueued; nothing is
// read back from the device.
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/kvq.h"
#include "kvq_launch.h"

namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

// Compute units of the current device (queried once per device).
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const kvq_cache *c) {
  if (c == nullptr) return KVQ_ERR_INVALID_ARG;
  if (c->page_size != 16 || c->num_pages <= 0) return KVQ_ERR_UNSUPPORTED;
  if (c->format == KVQ_FMT_E4M3) {
    if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if (c->num_kv_heads <= 0) return KVQ_ERR_INVALID_ARG;
    if (c->k == nullptr || c->v == nullptr) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(c->k) || !aligned16(c->v)) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
  }
  if (c->format == KVQ_FMT_NVFP4_MLA368) {
    if (c->head_dim != 576 || c->num_kv_heads != 1) return KVQ_ERR_UNSUPPORTED;
    if (c->k == nullptr || c->v != nullptr) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(c->k)) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
  }
  return KVQ_ERR_UNSUPPORTED;
}

int check_params(const kvq_cache *c, const kvq_attn_params *p) {
  if (p == nullptr) return KVQ_ERR_INVALID_ARG;
  if (p->num_q_heads <= 0 || p->num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  const uint32_t known = KVQ_FLAG_PREFILL_FP8_P | KVQ_FLAG_PREFILL_FP8_P2;
  if (p->window < 0 || p->num_splits < 0 || (p->flags & ~known) != 0 ||
      (p->flags & known) == known)
    return KVQ_ERR_INVALID_ARG;
  if (p->rel_bias != nullptr) {
    if (p->rel_extent < 1 || p->rel_extent > (1 << 20) || p->alibi_slopes != nullptr ||
        (reinterpret_cast<uintptr_t>(p->rel_bias) & 1) != 0)
      return KVQ_ERR_INVALID_ARG;
  } else if (p->rel_extent != 0) {
    return KVQ_ERR_INVALID_ARG;
  }
  if (!good_scale(p->softmax_scale) || !good_scale(p->k_scale)) return KVQ_ERR_BAD_SCALE;
  if (c->format == KVQ_FMT_E4M3 && (!good_scale(p->q_scale) || !good_scale(p->v_scale)))
    return KVQ_ERR_BAD_SCALE;
  if (c->format != KVQ_FMT_E4M3 && (p->window != 0 || p->alibi_slopes != nullptr || p->rel_bias != nullptr))
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// Split plan for the e4m3 decode kernel. Waves per workgroup and splits are
// chosen so the grid holds about 8 waves per compute unit, with at least one
// 128-key block per wave; sequences of up to 8 blocks run as one split.
kvq::DecodePlan plan_decode(const kvq_cache *c, int32_t num_seqs, int32_t max_seq_len,
                            const kvq_attn_params *p) {
  kvq::DecodePlan pl{};
  const int group = p->num_q_heads / c->num_kv_heads;
  pl.qtiles = (group + 15) / 16;
  const int64_t pages_full = (static_cast<int64_t>(max_seq_len) + 15) / 16;
  int64_t pages = pages_full;
  if (p->window > 0) {
    const int64_t wp = (static_cast<int64_t>(p->window) + 15) / 16 + 1;
    if (wp < pages) pages = wp;
  }
  const int64_t nblk = pages > 0 ? (pages + 7) / 8 : 1;
  const int64_t units = static_cast<int64_t>(num_seqs) * c->num_kv_heads * pl.qtiles;
  const int64_t target_waves = static_cast<int64_t>(current_cu_count()) * 8;
  // the smallest power of two of waves that gives each wave at most one block
  // of a short sequence (so one split suffices and no combine runs), else 8
  pl.waves = nblk > 4 ? 8 : (nblk > 2 ? 4 : (nblk > 1 ? 2 : 1));
  auto splits_for = [&](int64_t w) {
    int64_t sp = (target_waves + units * w - 1) / (units * w);
    const int64_t max_by_waves = (nblk + w - 1) / w;  // >= 1 block per wave
    return sp < max_by_waves ? sp : max_by_waves;
  };
  int64_t splits;
  if (p->num_splits > 0) {
    splits = p->num_splits;
  } else {
    splits = splits_for(pl.waves);
    // few (sequence, KV head) units over long sequences: fewer waves per
    // workgroup and more splits while the workgroups cover less than half of
    // the compute units (short sequences keep their single split: no
    // combine). Half is enough: the combine's cost grows with the split
    // count (one sequence over 65,536 keys on 2 KV heads: 64 splits of 8
    // waves 15.1 us per call, 128 of 4 waves 15.8, 256 of 2 waves 24.1)
    while (nblk > 8 && pl.waves > 1 && 2 * units * splits < current_cu_count()) {
      const int64_t s2 = splits_for(pl.waves / 2);
      if (s2 <= splits) break;
      pl.waves /= 2;
      splits = s2;
    }
  }
  if (splits > nblk) splits = nblk;
  if (splits < 1) splits = 1;
  pl.blocks_per_split = static_cast<int>((nblk + splits - 1) / splits);
  pl.splits = static_cast<int>((nblk + pl.blocks_per_split - 1) / pl.blocks_per_split);
  if (pl.splits == 1) {
    pl.workspace = 0;
  } else {
    const size_t rows = static_cast<size_t>(num_seqs) * p->num_q_heads * pl.splits;
    pl.workspace = rows * (static_cast<size_t>(c->head_dim) + 2) * sizeof(float);
  }
  return pl;
}

// NVFP4 decode: 64 splits of at most 512 pages
constexpr int64_t kMlaMaxSeqLen = 64 * 512 * 16;
constexpr int64_t kMlaPrefillMaxSeqLen = 2048 * 16;   // one split of the MLA kernel

kvq::MlaPlan plan_mla(int32_t num_seqs, int32_t max_seq_len, const kvq_attn_params *p) {
  kvq::MlaPlan pl{};
  const int64_t pages = max_seq_len > 0 ? (static_cast<int64_t>(max_seq_len) + 15) / 16 : 1;
  const int64_t target = static_cast<int64_t>(current_cu_count());   // one workgroup per CU
  int64_t splits = p->num_splits > 0 ? p->num_splits : (target + num_seqs - 1) / (num_seqs > 0 ? num_seqs : 1);
  // at least 4 pages (64 keys) per split, at most 512 (the kernel stages a
  // split's block-table slice in LDS); at most 64 splits (each adds a partial the combine reads)
  const int64_t max_splits = (pages + 3) / 4;
  if (splits > max_splits) splits = max_splits;
  if (splits > 64) splits = 64;
  if (splits < (pages + 511) / 512) splits = (pages + 511) / 512;
  if (splits < 1) splits = 1;
  pl.pages_per_split = static_cast<int>((pages + splits - 1) / splits);
  pl.splits = static_cast<int>((pages + pl.pages_per_split - 1) / pl.pages_per_split);
  if (pl.splits == 1) {
    pl.workspace = 0;
  } else {
    const size_t rows = static_cast<size_t>(num_seqs) * p->num_q_heads * pl.splits;
    pl.workspace = rows * (512 + 4) * sizeof(float);   // O partial, then (M, den, E, pad)
  }
  return pl;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// Per-block key norms of the slope-bias prefill: one float per (sequence,
// KV head, 128-key block).
size_t prefill_knorm_bytes(const kvq_cache *c, int32_t num_seqs, int32_t max_seq_len, const kvq_attn_params *p) {
  if (c->format != KVQ_FMT_E4M3 || p->alibi_slopes == nullptr || num_seqs <= 0 || max_seq_len <= 0) return 0;
  return static_cast<size_t>(num_seqs) * c->num_kv_heads * ((static_cast<size_t>(max_seq_len) + 127) / 128) *
         sizeof(float);
}

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char *kvq_status_str(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument (pointer, size, stride or alignment)";
    case KVQ_ERR_UNSUPPORTED: return "unsupported cache format or shape";
    case KVQ_ERR_BAD_SCALE: return "scale is not finite and positive";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_SCRATCH_LIMIT: return "split partials exceed the static scratch array (KVQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int kvq_store(const kvq_cache *cache, const void *k, int64_t k_token_stride, const void *v,
              int64_t v_token_stride, const int64_t *slot_mapping, int64_t num_tokens,
              float k_scale, float v_scale, kvq_stream_t stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (cache->format == KVQ_FMT_E4M3) {
    if (!good_scale(k_scale) || !good_scale(v_scale)) return KVQ_ERR_BAD_SCALE;
    if (num_tokens == 0) return KVQ_OK;
    const int64_t row = static_cast<int64_t>(cache->num_kv_heads) * cache->head_dim;
    if (k == nullptr || v == nullptr || slot_mapping == nullptr) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARG;
    if (k_token_stride < row || v_token_stride < row || k_token_stride % 8 || v_token_stride % 8)
      return KVQ_ERR_INVALID_ARG;
    kvq::StoreE4M3Launch a{};
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.k_stride = k_token_stride;
    a.v_stride = v_token_stride;
    a.slot = slot_mapping;
    a.num_tokens = num_tokens;
    a.kc = static_cast<uint8_t *>(cache->k);
    a.vc = static_cast<uint8_t *>(cache->v);
    a.hkv = cache->num_kv_heads;
    a.d = cache->head_dim;
    a.k_inv = 1.0f / k_scale;
    a.v_inv = 1.0f / v_scale;
    return hip_status(kvq::launch_store_e4m3(a, reinterpret_cast<hipStream_t>(stream)));
  }
  // NVFP4 record: k = [T][576] latent + RoPE, k_scale = RoPE scale
  if (!good_scale(k_scale)) return KVQ_ERR_BAD_SCALE;
  if (v != nullptr) return KVQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return KVQ_OK;
  if (k == nullptr || slot_mapping == nullptr || !aligned16(k)) return KVQ_ERR_INVALID_ARG;
  if (k_token_stride < 576 || k_token_stride % 8) return KVQ_ERR_INVALID_ARG;
  kvq::StoreNvfp4Launch a{};
  a.x = static_cast<const uint16_t *>(k);
  a.stride = k_token_stride;
  a.slot = slot_mapping;
  a.num_tokens = num_tokens;
  a.records = static_cast<uint8_t *>(cache->k);
  a.rope_inv = 1.0f / k_scale;
  a.static_s2 = 0.0f;
  return hip_status(kvq::launch_store_nvfp4(a, reinterpret_cast<hipStream_t>(stream)));
}

int kvq_store_nvfp4_static(const kvq_cache *cache, const void *x, int64_t token_stride,
                           const int64_t *slot_mapping, int64_t num_tokens, float rope_scale,
                           float outer_scale, kvq_stream_t stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->format != KVQ_FMT_NVFP4_MLA368) return KVQ_ERR_UNSUPPORTED;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (!good_scale(rope_scale) || !good_scale(outer_scale)) return KVQ_ERR_BAD_SCALE;
  if (num_tokens == 0) return KVQ_OK;
  if (x == nullptr || slot_mapping == nullptr || !aligned16(x)) return KVQ_ERR_INVALID_ARG;
  if (token_stride < 576 || token_stride % 8) return KVQ_ERR_INVALID_ARG;
  kvq::StoreNvfp4Launch a{};
  a.x = static_cast<const uint16_t *>(x);
  a.stride = token_stride;
  a.slot = slot_mapping;
  a.num_tokens = num_tokens;
  a.records = static_cast<uint8_t *>(cache->k);
  a.rope_inv = 1.0f / rope_scale;
  a.static_s2 = outer_scale;
  return hip_status(kvq::launch_store_nvfp4(a, reinterpret_cast<hipStream_t>(stream)));
}

int kvq_calibrate_amax(const void *x, int64_t num_rows, int64_t row_len, int64_t row_stride,
                       const int64_t *slot_mapping, float *amax_inout, float *scale_out,
                       kvq_stream_t stream) {
  if (amax_inout == nullptr || num_rows < 0 || row_len <= 0 || row_len % 8 || row_stride < row_len ||
      row_stride % 8)
    return KVQ_ERR_INVALID_ARG;
  if (num_rows > 0 && (x == nullptr || !aligned16(x))) return KVQ_ERR_INVALID_ARG;
  kvq::AmaxLaunch a{};
  a.x = static_cast<const uint16_t *>(x);
  a.rows = num_rows;
  a.row_len = row_len;
  a.row_stride = row_stride;
  a.slot = slot_mapping;
  a.amax_inout = amax_inout;
  a.scale_out = scale_out;
  return hip_status(kvq::launch_amax(a, current_cu_count(), reinterpret_cast<hipStream_t>(stream)));
}

int kvq_scale_from_amax(const float *amax, int32_t rule, float *scale_out, kvq_stream_t stream) {
  if (amax == nullptr || scale_out == nullptr || rule < KVQ_SCALE_AMAX_448 || rule > KVQ_SCALE_SAFETY_1P3)
    return KVQ_ERR_INVALID_ARG;
  return hip_status(kvq::launch_scale_rule(amax, rule, scale_out, reinterpret_cast<hipStream_t>(stream)));
}

int kvq_band_counts(const void *x, int64_t num_rows, int64_t row_len, int64_t row_stride,
                    const int64_t *slot_mapping, float scale, uint64_t *counts_inout, kvq_stream_t stream) {
  if (counts_inout == nullptr || (reinterpret_cast<uintptr_t>(counts_inout) & 7) != 0 || num_rows < 0 ||
      row_len <= 0 || row_len % 8 || row_stride < row_len || row_stride % 8)
    return KVQ_ERR_INVALID_ARG;
  if (!good_scale(scale)) return KVQ_ERR_BAD_SCALE;
  if (num_rows == 0) return KVQ_OK;
  if (x == nullptr || !aligned16(x)) return KVQ_ERR_INVALID_ARG;
  kvq::BandLaunch a{};
  a.x = static_cast<const uint16_t *>(x);
  a.rows = num_rows;
  a.row_len = row_len;
  a.row_stride = row_stride;
  a.slot = slot_mapping;
  a.inv = 1.0f / scale;
  a.counts = reinterpret_cast<unsigned long long *>(counts_inout);
  return hip_status(kvq::launch_band_counts(a, current_cu_count(), reinterpret_cast<hipStream_t>(stream)));
}

size_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t num_seqs, int32_t max_seq_len,
                                  const kvq_attn_params *params) {
  if (check_cache(cache) != KVQ_OK || check_params(cache, params) != KVQ_OK) return 0;
  if (num_seqs <= 0 || max_seq_len < 0) return 0;
  if (cache->format == KVQ_FMT_E4M3) return plan_decode(cache, num_seqs, max_seq_len, params).workspace;
  return plan_mla(num_seqs, max_seq_len, params).workspace;
}

}  // extern "C"

namespace kvq {

int decode_check(const kvq_cache *cache, const void *q, const void *k_new, const void *v_new,
                 const int32_t *block_table, int64_t block_table_stride, const int32_t *seq_lens,
                 int32_t num_seqs, int32_t max_seq_len, const kvq_attn_params *params, void *out,
                 size_t *workspace_needed) {
  *workspace_needed = 0;
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  st = check_params(cache, params);
  if (st != KVQ_OK) return st;
  const bool append = k_new != nullptr || v_new != nullptr;
  if (append && cache->format != KVQ_FMT_E4M3) return KVQ_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_seq_len < 0) return KVQ_ERR_INVALID_ARG;
  if (num_seqs == 0) return KVQ_OK;
  if (append && (k_new == nullptr || v_new == nullptr || !aligned16(k_new) || !aligned16(v_new)))
    return KVQ_ERR_INVALID_ARG;
  if (q == nullptr || block_table == nullptr || seq_lens == nullptr || out == nullptr) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (block_table_stride * 16 < max_seq_len) return KVQ_ERR_INVALID_ARG;
  if (cache->format == KVQ_FMT_E4M3) {
    *workspace_needed = plan_decode(cache, num_seqs, max_seq_len, params).workspace;
    return KVQ_OK;
  }
  if (params->num_q_heads != 16) return KVQ_ERR_UNSUPPORTED;
  if (max_seq_len > kMlaMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
  *workspace_needed = plan_mla(num_seqs, max_seq_len, params).workspace;
  return KVQ_OK;
}

int decode_run(const kvq_cache *cache, const void *q, const void *k_new, const void *v_new,
               const int32_t *block_table, int64_t block_table_stride, const int32_t *seq_lens,
               int32_t num_seqs, int32_t max_seq_len, const kvq_attn_params *params, void *out,
               void *workspace, size_t workspace_bytes, kvq_stream_t stream) {
  size_t need = 0;
  int st = decode_check(cache, q, k_new, v_new, block_table, block_table_stride, seq_lens, num_seqs,
                        max_seq_len, params, out, &need);
  if (st != KVQ_OK || num_seqs == 0) return st;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return KVQ_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return KVQ_ERR_INVALID_ARG;
  const bool append = k_new != nullptr || v_new != nullptr;
  if (cache->format == KVQ_FMT_E4M3) {
    const kvq::DecodePlan pl = plan_decode(cache, num_seqs, max_seq_len, params);
    kvq::DecodeE4M3Launch a{};
    a.q = static_cast<const uint16_t *>(q);
    a.kc = static_cast<const uint8_t *>(cache->k);
    a.vc = static_cast<const uint8_t *>(cache->v);
    a.block_table = block_table;
    a.bt_stride = block_table_stride;
    a.seq_lens = seq_lens;
    a.slopes = params->alibi_slopes;
    a.rel = params->rel_bias;
    a.rel_extent = params->rel_extent;
    a.out = static_cast<uint16_t *>(out);
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = pl.workspace > 0
                    ? static_cast<float *>(workspace) +
                          static_cast<size_t>(num_seqs) * params->num_q_heads * pl.splits * cache->head_dim
                    : nullptr;
    a.batch = num_seqs;
    a.hq = params->num_q_heads;
    a.hkv = cache->num_kv_heads;
    a.d = cache->head_dim;
    a.window = params->window;
    a.q_inv = 1.0f / params->q_scale;
    a.fold_log2 = params->softmax_scale * params->q_scale * params->k_scale * 1.4426950408889634f;
    a.v_scale = params->v_scale;
    if (append) {
      a.k_new = static_cast<const uint16_t *>(k_new);
      a.v_new = static_cast<const uint16_t *>(v_new);
      a.kc_w = static_cast<uint8_t *>(cache->k);
      a.vc_w = static_cast<uint8_t *>(cache->v);
      a.k_inv = 1.0f / params->k_scale;   // as kvq_store computes them
      a.v_inv = 1.0f / params->v_scale;
    }
    return hip_status(kvq::launch_decode_e4m3(a, pl, reinterpret_cast<hipStream_t>(stream)));
  }
  const kvq::MlaPlan pl = plan_mla(num_seqs, max_seq_len, params);
  kvq::DecodeMlaLaunch a{};
  a.q = static_cast<const uint16_t *>(q);
  a.records = static_cast<const uint8_t *>(cache->k);
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t *>(out);
  a.part_o = static_cast<float *>(workspace);
  a.part_ml = pl.workspace > 0
                  ? static_cast<float *>(workspace) + static_cast<size_t>(num_seqs) * params->num_q_heads * pl.splits * 512
                  : nullptr;
  a.batch = num_seqs;
  a.hq = params->num_q_heads;
  a.scale_log2 = params->softmax_scale * 1.4426950408889634f;
  a.rope_scale = params->k_scale;
  return hip_status(kvq::launch_decode_mla(a, pl, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace kvq

extern "C" {

int kvq_paged_attn_decode(const kvq_cache *cache, const void *q, const int32_t *block_table,
                          int64_t block_table_stride, const int32_t *seq_lens, int32_t num_seqs,
                          int32_t max_seq_len, const kvq_attn_params *params, void *out,
                          void *workspace, size_t workspace_bytes, kvq_stream_t stream) {
  return kvq::decode_run(cache, q, nullptr, nullptr, block_table, block_table_stride, seq_lens, num_seqs,
                     max_seq_len, params, out, workspace, workspace_bytes, stream);
}

int kvq_paged_attn_decode_append(const kvq_cache *cache, const void *q, const void *k_new,
                                 const void *v_new, const int32_t *block_table,
                                 int64_t block_table_stride, const int32_t *seq_lens,
                                 int32_t num_seqs, int32_t max_seq_len,
                                 const kvq_attn_params *params, void *out, void *workspace,
                                 size_t workspace_bytes, kvq_stream_t stream) {
  if (k_new == nullptr || v_new == nullptr) return KVQ_ERR_INVALID_ARG;
  return kvq::decode_run(cache, q, k_new, v_new, block_table, block_table_stride, seq_lens, num_seqs,
                     max_seq_len, params, out, workspace, workspace_bytes, stream);
}

size_t kvq_prefill_workspace_bytes(const kvq_cache *cache, int32_t num_seqs, int32_t max_seq_len,
                                   const kvq_attn_params *params) {
  if (check_cache(cache) != KVQ_OK || check_params(cache, params) != KVQ_OK || num_seqs < 0 || max_seq_len < 0)
    return 0;
  return prefill_knorm_bytes(cache, num_seqs, max_seq_len, params);
}

int kvq_paged_attn_prefill(const kvq_cache *cache, const void *q, const int32_t *cu_q_lens, int64_t total_q,
                           int32_t max_q_len, const int32_t *block_table, int64_t block_table_stride,
                           const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len,
                           const kvq_attn_params *params, void *out, void *workspace,
                           size_t workspace_bytes, kvq_stream_t stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->format == KVQ_FMT_E4M3 && cache->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  st = check_params(cache, params);
  if (st != KVQ_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || total_q < 0 || max_q_len < 0) return KVQ_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return KVQ_OK;
  if (q == nullptr || cu_q_lens == nullptr || block_table == nullptr || seq_lens == nullptr || out == nullptr)
    return KVQ_ERR_INVALID_ARG;
  if (!aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (block_table_stride * 16 < max_seq_len || max_q_len > max_seq_len) return KVQ_ERR_INVALID_ARG;
  if (cache->format != KVQ_FMT_E4M3) {
    if (params->num_q_heads != 16 || max_seq_len > kMlaPrefillMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
    if (max_q_len == 0) return KVQ_OK;
    kvq::DecodeMlaLaunch m{};
    m.q = static_cast<const uint16_t *>(q);
    m.records = static_cast<const uint8_t *>(cache->k);
    m.block_table = block_table;
    m.bt_stride = block_table_stride;
    m.seq_lens = seq_lens;
    m.out = static_cast<uint16_t *>(out);
    m.batch = num_seqs;
    m.hq = params->num_q_heads;
    m.scale_log2 = params->softmax_scale * 1.4426950408889634f;
    m.rope_scale = params->k_scale;
    m.cu_q_lens = cu_q_lens;
    m.max_q_len = max_q_len;
    return hip_status(kvq::launch_prefill_mla(m, max_seq_len, reinterpret_cast<hipStream_t>(stream)));
  }
  kvq::PrefillE4M3Launch a{};
  a.q = static_cast<const uint16_t *>(q);
  a.cu_q_lens = cu_q_lens;
  a.kc = static_cast<const uint8_t *>(cache->k);
  a.vc = static_cast<const uint8_t *>(cache->v);
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.slopes = params->alibi_slopes;
  a.rel = params->rel_bias;
  a.rel_extent = params->rel_extent;
  a.out = static_cast<uint16_t *>(out);
  a.batch = num_seqs;
  a.hq = params->num_q_heads;
  a.hkv = cache->num_kv_heads;
  a.d = cache->head_dim;
  a.window = params->window;
  a.max_q_len = max_q_len;
  a.p_mode = (params->flags & KVQ_FLAG_PREFILL_FP8_P) != 0 ? 1 : ((params->flags & KVQ_FLAG_PREFILL_FP8_P2) != 0 ? 2 : 0);
  a.q_inv = 1.0f / params->q_scale;
  a.fold_log2 = params->softmax_scale * params->q_scale * params->k_scale * 1.4426950408889634f;
  a.v_scale = params->v_scale;
  const size_t knorm_bytes = prefill_knorm_bytes(cache, num_seqs, max_seq_len, params);
  if (knorm_bytes > 0 && workspace != nullptr && workspace_bytes >= knorm_bytes &&
      (reinterpret_cast<uintptr_t>(workspace) & 3) == 0) {
    a.knorm = static_cast<float *>(workspace);
    a.knorm_blocks = static_cast<int>((static_cast<int64_t>(max_seq_len) + 127) / 128);
  }
  return hip_status(kvq::launch_prefill_e4m3(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
