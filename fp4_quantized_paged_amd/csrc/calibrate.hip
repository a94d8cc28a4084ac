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
  int64_t r = ((int64_t)blockIdx.x * kAmaxWaves + wave) * kRowUnroll;
  // each wave takes kRowUnroll consecutive rows per iteration (a workgroup
  // reads one contiguous span), several loads per lane in flight
  for (; r < a.rows; r += nwaves * kRowUnroll) {
    uint4 x[kRowUnroll];
    bool keep[kRowUnroll];
    for (int64_t c = lane; c < cpr; c += 64) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t rr = r + u;
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

// Scale rules (vLLM PR 54705 evidence "Tier 4": max(1, amax * 1.3 / 448);
// model card "Rebuild / reproduce": ceil_to_bfloat16(amax / 448)).
__global__ void scale_rule_kernel(const float *amax, int rule, float *scale) {
  if (threadIdx.x != 0) return;
  const float a = amax[0];
  float s;
  if (rule == 0) {
    s = a / kE4M3Max;
  } else if (rule == 1) {
    uint32_t b = __float_as_uint(a / kE4M3Max);
    if (b & 0xFFFFu) b = (b & 0xFFFF0000u) + 0x10000u;   // up to the next bf16
    s = __uint_as_float(b);
  } else {
    const double t = (double)a * 1.3 / 448.0;
    s = (float)(t > 1.0 ? t : 1.0);                        // NaN -> 1, as max(1, NaN)
  }
  scale[0] = s;
}

// Band counters (vLLM PR 54705 evidence "Tier 2": clip and flush-to-zero
// counts of the stored values at a scale). Each value is decided with the
// store's own arithmetic: y = fp32(x) * inv; clipped when |y| > 448 (the
// clamp changes it; NaN compares false); flushed when the bf16 input is
// nonzero and not NaN and its e4m3 code is +-0. Both decisions are monotone
// in |x|, and non-negative bf16 values order like their bit patterns, so
// each band is a range of magnitude patterns: clipped (T, 0x7F80] (0x7F80 is
// inf), flushed [1, F], with T and F found once per thread by bisection on
// that same arithmetic (the store's multiply and its hardware conversion).
// Per-lane counts, one wave and workgroup reduction, two 64-bit atomic adds
// per workgroup.
__device__ __forceinline__ float bf16_mag(uint32_t m) { return __uint_as_float(m << 16); }

__global__ __launch_bounds__(kAmaxThreads) void band_kernel(BandLaunch a) {
  __shared__ uint32_t red[2][kAmaxWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t cpr = a.row_len >> 3;
  const int64_t nwaves = (int64_t)gridDim.x * kAmaxWaves;
  // T: the largest magnitude that the clamp leaves alone (0 does, inf does not)
  uint32_t lo = 0, hi = 0x7F80u;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (fabsf(bf16_mag(mid) * a.inv) > kE4M3Max) hi = mid; else lo = mid;
  }
  const uint32_t clip_span = 0x7F80u - lo;   // clipped: mag - (T + 1) < clip_span
  const uint32_t clip_lo = lo + 1;
  // F: the largest magnitude whose e4m3 code is zero (0 is, 448 / inv is not)
  lo = 0;
  hi = 0x7F80u;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    const float y = sat448(bf16_mag(mid) * a.inv);
    if ((cvt4_e4m3(y, 0.0f, 0.0f, 0.0f) & 0x7Fu) != 0) hi = mid; else lo = mid;
  }
  const uint32_t flush_hi = lo;              // flushed: mag - 1 < F
  uint32_t n_clip = 0, n_flush = 0;
  int64_t r = ((int64_t)blockIdx.x * kAmaxWaves + wave) * kRowUnroll;
  for (; r < a.rows; r += nwaves * kRowUnroll) {
    for (int64_t c = lane; c < cpr; c += 64) {
      uint4 x[kRowUnroll];
      bool keep[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t rr = r + u;
        keep[u] = rr < a.rows && (a.slot == nullptr || a.slot[rr] >= 0);
        if (keep[u]) {
          const v4u w = __builtin_nontemporal_load((const v4u *)(a.x + rr * a.row_stride + (c << 3)));
          x[u] = make_uint4(w.x, w.y, w.z, w.w);
        } else {
          x[u] = make_uint4(0, 0, 0, 0);   // zeros count in neither band
        }
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const uint32_t wd[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t mag = (wd[e >> 1] >> (16 * (e & 1))) & 0x7FFFu;
          n_clip += (mag - clip_lo < clip_span) ? 1u : 0u;
          n_flush += (mag - 1u < flush_hi) ? 1u : 0u;
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    n_clip += (uint32_t)__shfl_xor((int)n_clip, off, 64);
    n_flush += (uint32_t)__shfl_xor((int)n_flush, off, 64);
  }
  if (lane == 0) {
    red[0][wave] = n_clip;
    red[1][wave] = n_flush;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t0 = 0, t1 = 0;
#pragma unroll
    for (int i = 0; i < kAmaxWaves; ++i) {
      t0 += red[0][i];
      t1 += red[1][i];
    }
    if (t0) atomicAdd(a.counts, t0);
    if (t1) atomicAdd(a.counts + 1, t1);
  }
}

}  // namespace

hipError_t launch_amax(const AmaxLaunch &a, int num_cus, hipStream_t s) {
  if (a.rows > 0) {
    // a load-only stream: 4 workgroups (16 waves) per CU with four 16-byte
    // loads per lane in flight measured fastest (more waves, or a second
    // round of workgroups, streamed slower)
    int64_t blocks = (a.rows + kAmaxWaves * kRowUnroll - 1) / (kAmaxWaves * kRowUnroll);
    const int64_t cap = (int64_t)num_cus * 4;
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

hipError_t launch_scale_rule(const float *amax, int rule, float *scale, hipStream_t s) {
  hipLaunchKernelGGL(scale_rule_kernel, dim3(1), dim3(64), 0, s, amax, rule, scale);
  return hipGetLastError();
}

hipError_t launch_band_counts(const BandLaunch &a, int num_cus, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  int64_t blocks = (a.rows + kAmaxWaves * kRowUnroll - 1) / (kAmaxWaves * kRowUnroll);
  // 4 workgroups per CU, as for amax (a sweep of 4 / 8 / 16 / 32 per CU
  // measured 174 / 180 / 196 / 226 us over the batched-decode K and V)
  const int64_t cap = (int64_t)num_cus * 4;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(band_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
