// kvq_paged_attn_decode_noalloc: the paged decode with its split partials in
// a static device array instead of a caller workspace, for callers that
// cannot allocate device memory (graph capture, serving loops, harnesses
// that forbid hipMalloc). Same kernels and split plan as
// kvq_paged_attn_decode.
#include <mutex>

#include "../../include/kvq.h"
#include "kvq_launch.h"

namespace {

// The split partials of every no-alloc call on a device. In host code
// `scratch` is only a handle for the runtime's symbol lookup: kernels get the
// device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// This device's copy of `scratch`, looked up once per device with the device
// current. Returns nullptr if the lookup failed.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev]() {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" int kvq_paged_attn_decode_noalloc(const kvq_cache *cache, const void *q,
                                             const int32_t *block_table, int64_t block_table_stride,
                                             const int32_t *seq_lens, int32_t num_seqs,
                                             int32_t max_seq_len, const kvq_attn_params *params,
                                             void *out, kvq_stream_t stream) {
  size_t need = 0;
  const int st = kvq::decode_check(cache, q, nullptr, nullptr, block_table, block_table_stride, seq_lens,
                                   num_seqs, max_seq_len, params, out, &need);
  if (st != KVQ_OK || num_seqs == 0) return st;
  if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (ws == nullptr) return KVQ_ERR_HIP;
  }
  return kvq::decode_run(cache, q, nullptr, nullptr, block_table, block_table_stride, seq_lens, num_seqs,
                         max_seq_len, params, out, ws, need > 0 ? KVQ_NOALLOC_SCRATCH_BYTES : 0, stream);
}
