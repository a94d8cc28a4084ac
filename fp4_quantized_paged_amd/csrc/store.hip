// Quant-on-store of bf16 K/V into the paged e4m3 cache.
//
// vLLM PR 54705, "Purpose" (quant-on-store bullet): K/V are quantized to the
// cache dtype as they are written, with a clamp to the e4m3 finite range
// because a plain float-to-fp8 store does not saturate; evidence "Tier 1"
// (write path): the added work is a multiply, a clamp and a convert, paid for
// by halved write bytes.
//
// One workgroup handles 16 consecutive input tokens. When those 16 tokens fill
// one page in order (the bulk-prefill case), the token-minor V page image is
// assembled in LDS and written with 16-byte stores; otherwise (decode append,
// ragged or scattered slots) each token is written in place.
#include "kvq_device.h"
#include "kvq_launch.h"

#pragma clang fp contract(off)

namespace kvq {

namespace {

constexpr int kStoreThreads = 256;

__global__ __launch_bounds__(kStoreThreads) void store_e4m3_kernel(StoreE4M3Launch a, int use_lds) {
  extern __shared__ __align__(16) uint8_t vimg[];   // [hkv][d][16] when use_lds
  __shared__ int s_fast;
  __shared__ int64_t s_page;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kPage;
  const int ntok = (int)min<int64_t>(kPage, a.num_tokens - t0);
  const int row = a.hkv * a.d;        // elements per token
  const int cpr = row >> 3;           // 8-element chunks per token
  const int cpd = a.d >> 3;           // chunks per head row

  if (tid < 64) {
    const int i = tid;
    int64_t s = (i < ntok) ? a.slot[t0 + i] : -1;
    const int64_t s0 = __shfl(s, 0, 64);
    const bool ok = (i >= kPage) || (ntok == kPage && s0 >= 0 && (s0 & (kPage - 1)) == 0 && s == s0 + i);
    const uint64_t bal = __ballot(ok);
    if (tid == 0) {
      s_fast = use_lds && (bal == ~0ull);
      s_page = s0 >> 4;
    }
  }
  __syncthreads();

  if (s_fast) {
    const int64_t page = s_page;
    uint8_t *kpage = a.kc + (size_t)page * (size_t)row * kPage;
    for (int c = tid; c < kPage * cpr; c += kStoreThreads) {
      const int i = c / cpr;
      const int r = c - i * cpr;
      const int h = r / cpd;
      const int d0 = (r - h * cpd) << 3;
      const uint4 kx = *(const uint4 *)(a.k + (t0 + i) * a.k_stride + (r << 3));
      const uint4 vx = *(const uint4 *)(a.v + (t0 + i) * a.v_stride + (r << 3));
      const uint2 kq = quant8_e4m3(kx, a.k_inv);
      const uint2 vq = quant8_e4m3(vx, a.v_inv);
      *(uint2 *)(kpage + ((size_t)(h * kPage + i) * a.d + d0)) = kq;
      uint8_t *dst = vimg + (size_t)(h * a.d + d0) * kPage + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[j * kPage] = (uint8_t)(vq.x >> (8 * j));
        dst[(j + 4) * kPage] = (uint8_t)(vq.y >> (8 * j));
      }
    }
    __syncthreads();
    uint4 *vdst = (uint4 *)(a.vc + (size_t)page * (size_t)row * kPage);
    const uint4 *vsrc = (const uint4 *)vimg;
    for (int c = tid; c < row; c += kStoreThreads) vdst[c] = vsrc[c];  // row*16 bytes
    return;
  }

  for (int c = tid; c < ntok * cpr; c += kStoreThreads) {
    const int i = c / cpr;
    const int r = c - i * cpr;
    const int64_t s = a.slot[t0 + i];
    if (s < 0) continue;
    const int h = r / cpd;
    const int d0 = (r - h * cpd) << 3;
    const int64_t page = s >> 4;
    const int off = (int)(s & (kPage - 1));
    const uint4 kx = *(const uint4 *)(a.k + (t0 + i) * a.k_stride + (r << 3));
    const uint4 vx = *(const uint4 *)(a.v + (t0 + i) * a.v_stride + (r << 3));
    const uint2 kq = quant8_e4m3(kx, a.k_inv);
    const uint2 vq = quant8_e4m3(vx, a.v_inv);
    *(uint2 *)(a.kc + (((size_t)page * a.hkv + h) * kPage + off) * a.d + d0) = kq;
    uint8_t *dst = a.vc + (((size_t)page * a.hkv + h) * a.d + d0) * kPage + off;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[j * kPage] = (uint8_t)(vq.x >> (8 * j));
      dst[(j + 4) * kPage] = (uint8_t)(vq.y >> (8 * j));
    }
  }
}

}  // namespace

hipError_t launch_store_e4m3(const StoreE4M3Launch &a, hipStream_t s) {
  const int64_t blocks = (a.num_tokens + kPage - 1) / kPage;
  const size_t img = (size_t)a.hkv * a.d * kPage;
  const int use_lds = img <= 64 * 1024;
  hipLaunchKernelGGL(store_e4m3_kernel, dim3((unsigned)blocks), dim3(kStoreThreads),
                     use_lds ? img : 0, s, a, use_lds);
  return hipGetLastError();
}

}  // namespace kvq
