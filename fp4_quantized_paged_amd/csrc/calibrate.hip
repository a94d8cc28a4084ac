// amax calibration: running max |x| over stored rows and scale = amax / 448.
//
// Qwen3.8-27B-FP8-KVcal model card: the k, v and q scales are amax/448 of the
// values observed at the cache-write point ("Observation point", scale table);
// the calibration hook keeps a running |K|/|V| amax across calls ("Rebuild /
// reproduce"). vLLM PR 54705 evidence "Tier 2": statistics must cover exactly
// the stored values, so rows whose slot is negative (not stored) are skipped.
//
// |bf16| orders like its bit pattern with the sign cleared, so the maximum is
// an integer max: exact and independent of reduction order. Each wave walks
// whole rows (one 16-byte load per lane per 8 elements), reduces across the
// wave and the workgroup, and issues one atomic max on the fp32 bit pattern
// of the running amax. A one-thread kernel then writes amax / 448.
#include "kvq_device.h"
#include "kvq_launch.h"

#pragma clang fp contract(off)

namespace kvq {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxWaves = kAmaxThreads / 64;
constexpr int kRowUnroll = 4;

__device__ __forceinline__ uint32_t absmax_u4(uint4 x, uint32_t m) {
  const uint32_t a = max(x.x & 0x7FFFu, (x.x >> 16) & 0x7FFFu);
  const uint32_t b = max(x.y & 0x7FFFu, (x.y >> 16) & 0x7FFFu);
  const uint32_t c = max(x.z & 0x7FFFu, (x.z >> 16) & 0x7FFFu);
  const uint32_t d = max(x.w & 0x7FFFu, (x.w >> 16) & 0x7FFFu);
  return max(m, max(max(a, b), max(c, d)));
}

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(AmaxLaunch a) {
  __shared__ uint32_t red[kAmaxWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t cpr = a.row_len >> 3;
  const int64_t nwaves = (int64_t)gridDim.x * kAmaxWaves;
  uint32_t m = 0;
  int64_t r = (int64_t)blockIdx.x * kAmaxWaves + wave;
  // kRowUnroll rows per iteration keep several loads per lane in flight
  for (; r < a.rows; r += nwaves * kRowUnroll) {
    uint4 x[kRowUnroll];
    bool keep[kRowUnroll];
    for (int64_t c = lane; c < cpr; c += 64) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t rr = r + u * nwaves;
        keep[u] = rr < a.rows && (a.slot == nullptr || a.slot[rr] >= 0);
        if (keep[u]) {
          const v4u w = __builtin_nontemporal_load((const v4u *)(a.x + rr * a.row_stride + (c << 3)));
          x[u] = make_uint4(w.x, w.y, w.z, w.w);
        } else {
          x[u] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) m = absmax_u4(x[u], m);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = red[0];
#pragma unroll
    for (int i = 1; i < kAmaxWaves; ++i) w = max(w, red[i]);
    if (w) atomicMax((unsigned int *)a.amax_inout, w << 16);
  }
}

__global__ void amax_finalize_kernel(const float *amax, float *scale) {
  if (threadIdx.x == 0) scale[0] = amax[0] / kE4M3Max;
}

}  // namespace

hipError_t launch_amax(const AmaxLaunch &a, int num_cus, hipStream_t s) {
  if (a.rows > 0) {
    int64_t blocks = (a.rows + kAmaxWaves * kRowUnroll - 1) / (kAmaxWaves * kRowUnroll);
    const int64_t cap = (int64_t)num_cus * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.scale_out) {
    hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(64), 0, s, a.amax_inout, a.scale_out);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kvq
