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
// assembled in LDS and leaves in contiguous 16-byte stores (every store
// instruction writes whole lines); otherwise (decode append, ragged or
// scattered slots) each token is written in place, its V bytes passing
// through LDS so that each byte-store instruction covers few lines.
#include "kvq_device.h"
#include "kvq_launch.h"

#pragma clang fp contract(off)

namespace kvq {

namespace {

constexpr int kStoreThreads = 256;
constexpr int kUnroll = 2;   // 16-element chunks per thread per round

// Streaming (non-temporal) loads and stores: every byte is touched once.
__device__ __forceinline__ uint4 ld_nt16(const uint16_t *p) {
  const v4u x = __builtin_nontemporal_load((const v4u *)p);
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_nt16(uint8_t *p, uint2 lo, uint2 hi) {
  __builtin_nontemporal_store(v4u{lo.x, lo.y, hi.x, hi.y}, (v4u *)p);
}

// 16 consecutive bf16 elements of one token (two 16-byte loads).
struct Chunk {
  uint4 k0, k1, v0, v1;
};

__device__ __forceinline__ void load_chunk(const StoreE4M3Launch &a, int64_t t, int e0, Chunk &c) {
  const uint16_t *kp = a.k + t * a.k_stride + e0;
  const uint16_t *vp = a.v + t * a.v_stride + e0;
  c.k0 = ld_nt16(kp);
  c.k1 = ld_nt16(kp + 8);
  c.v0 = ld_nt16(vp);
  c.v1 = ld_nt16(vp + 8);
}

__global__ __launch_bounds__(kStoreThreads) void store_e4m3_kernel(StoreE4M3Launch a, int use_lds) {
  extern __shared__ __align__(16) uint8_t vimg[];   // when use_lds: [16][hkv*d] V bytes, then [hkv*d][16]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * kPage;
  const int ntok = (int)min<int64_t>(kPage, a.num_tokens - t0);
  const int row = a.hkv * a.d;        // elements per token
  const int cpr = row >> 4;           // 16-element chunks per token
  const int cpd = a.d >> 4;           // chunks per head row
  const int nchunk = ntok * cpr;

  // Lane i < 16 of every wave holds the slot of token t0 + i. The inputs of
  // the first kUnroll chunks are requested in the same round trip.
  const int64_t my_slot = lane < ntok ? a.slot[t0 + lane] : -1;
  Chunk ch[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int c = tid + u * kStoreThreads;
    const int i = c / cpr;
    if (c < nchunk) load_chunk(a, t0 + i, (c - i * cpr) << 4, ch[u]);
  }
  // Whole page in order? Every wave derives the same answer from the same
  // 16 slots, so the branch is uniform over the workgroup.
  const int64_t s0 = __shfl(my_slot, 0, 64);
  const bool ok = lane >= kPage ||
                  (ntok == kPage && s0 >= 0 && (s0 & (kPage - 1)) == 0 && my_slot == s0 + lane);
  const bool fast = use_lds && __ballot(ok) == ~0ull;

  if (fast) {
    // Stage 1: quantize; K rows go straight to the page, V bytes land
    // token-major in LDS ([16 tokens][row], 16-byte writes).
    const int64_t page = s0 >> 4;
    uint8_t *kpage = a.kc + (size_t)page * (size_t)row * kPage;
    for (int c0 = 0; c0 < nchunk; c0 += kStoreThreads * kUnroll) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + tid + u * kStoreThreads;
          const int i = c / cpr;
          if (c < nchunk) load_chunk(a, t0 + i, (c - i * cpr) << 4, ch[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + tid + u * kStoreThreads;
        if (c >= nchunk) break;
        const int i = c / cpr;
        const int r = c - i * cpr;
        const int h = r / cpd;
        const int d0 = (r - h * cpd) << 4;
        st_nt16(kpage + ((size_t)(h * kPage + i) * a.d + d0), quant8_e4m3(ch[u].k0, a.k_inv),
                quant8_e4m3(ch[u].k1, a.k_inv));
        const uint2 v0 = quant8_e4m3(ch[u].v0, a.v_inv), v1 = quant8_e4m3(ch[u].v1, a.v_inv);
        *(uint4 *)(vimg + (size_t)i * row + (r << 4)) = make_uint4(v0.x, v0.y, v1.x, v1.y);
      }
    }
    __syncthreads();
    // Stage 2: each thread takes 4 adjacent columns (head*D + dim) of the 16
    // tokens, transposes the 16x4 bytes in registers and writes four 16-byte
    // token-minor rows to the second LDS image ([head][dim][16], the V page).
    uint8_t *vmin = vimg + (size_t)kPage * row;
    for (int q4 = tid; q4 < (row >> 2); q4 += kStoreThreads) {
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = *(const uint32_t *)(vimg + (size_t)i * row + 4 * q4);
      uint32_t o[4][4];   // o[b][blk]: column 4*q4+b, tokens 4*blk .. 4*blk+3
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const uint32_t w0 = w[4 * blk], w1 = w[4 * blk + 1], w2 = w[4 * blk + 2], w3 = w[4 * blk + 3];
        const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // w0.0 w1.0 w0.1 w1.1
        const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // w0.2 w1.2 w0.3 w1.3
        const uint32_t t2 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
        const uint32_t t3 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
        o[0][blk] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);          // w0.0 w1.0 w2.0 w3.0
        o[1][blk] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
        o[2][blk] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
        o[3][blk] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) *(v4u *)(vmin + (size_t)(4 * q4 + b) * kPage) = v4u{o[b][0], o[b][1], o[b][2], o[b][3]};
    }
    __syncthreads();
    // Stage 3: the page image leaves with consecutive lanes on consecutive
    // 16-byte rows.
    uint8_t *vpage = a.vc + (size_t)page * (size_t)row * kPage;
    for (int c = tid; c < row; c += kStoreThreads)
      __builtin_nontemporal_store(*(const v4u *)(vmin + (size_t)c * kPage), (v4u *)(vpage + (size_t)c * kPage));
    return;
  }

  if (use_lds) {
    // Scattered slots (decode append, ragged tails): K chunks go to their rows
    // in place (16-byte stores); V bytes are staged token-major in LDS and
    // then leave one byte per lane, consecutive lanes on consecutive dims of
    // one token, so a store instruction covers 8 lines (a 16-byte stride)
    // rather than 64. The slot of token i comes from lane i of each wave.
    for (int c0 = 0; c0 < nchunk; c0 += kStoreThreads * kUnroll) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + tid + u * kStoreThreads;
          const int i = c / cpr;
          if (c < nchunk) load_chunk(a, t0 + i, (c - i * cpr) << 4, ch[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + tid + u * kStoreThreads;
        const int i = min(c / cpr, kPage - 1);
        const int64_t sl = __shfl(my_slot, i, 64);
        if (c >= nchunk) continue;
        const int r = c - i * cpr;
        const uint2 v0 = quant8_e4m3(ch[u].v0, a.v_inv), v1 = quant8_e4m3(ch[u].v1, a.v_inv);
        *(uint4 *)(vimg + (size_t)i * row + (r << 4)) = make_uint4(v0.x, v0.y, v1.x, v1.y);
        if (sl < 0) continue;
        const int h = r / cpd;
        const int d0 = (r - h * cpd) << 4;
        const uint2 k0 = quant8_e4m3(ch[u].k0, a.k_inv), k1 = quant8_e4m3(ch[u].k1, a.k_inv);
        *(uint4 *)(a.kc + ((((size_t)(sl >> 4)) * a.hkv + h) * kPage + (sl & (kPage - 1))) * a.d + d0) =
            make_uint4(k0.x, k0.y, k1.x, k1.y);
      }
    }
    __syncthreads();
    // one token per wave at a time: column col = head * d + dim of the token
    // lands at byte 16 * col + (slot & 15) of its page
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = wave; i < ntok; i += kStoreThreads / 64) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_slot, i);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)my_slot >> 32), i);
      const int64_t sl = (int64_t)(((uint64_t)hi << 32) | lo);
      if (sl < 0) continue;
      uint8_t *dst = a.vc + (size_t)(sl >> 4) * (size_t)row * kPage + (sl & (kPage - 1));
      const uint8_t *src = vimg + (size_t)i * row;
#pragma unroll 8
      for (int col = lane; col < row; col += 64) dst[(size_t)col * kPage] = src[col];
    }
    return;
  }

  // Rows too wide for the LDS image: each chunk is written in place.
  for (int c0 = 0; c0 < nchunk; c0 += kStoreThreads * kUnroll) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + tid + u * kStoreThreads;
        const int i = c / cpr;
        if (c < nchunk) load_chunk(a, t0 + i, (c - i * cpr) << 4, ch[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + tid + u * kStoreThreads;
      const int i = min(c / cpr, kPage - 1);
      const int64_t sl = __shfl(my_slot, i, 64);
      if (c >= nchunk || sl < 0) continue;
      const int r = c - i * cpr;
      const int h = r / cpd;
      const int d0 = (r - h * cpd) << 4;
      const int64_t page = sl >> 4;
      const int off = (int)(sl & (kPage - 1));
      const uint2 k0 = quant8_e4m3(ch[u].k0, a.k_inv), k1 = quant8_e4m3(ch[u].k1, a.k_inv);
      *(uint4 *)(a.kc + (((size_t)page * a.hkv + h) * kPage + off) * a.d + d0) = make_uint4(k0.x, k0.y, k1.x, k1.y);
      const uint2 v0 = quant8_e4m3(ch[u].v0, a.v_inv), v1 = quant8_e4m3(ch[u].v1, a.v_inv);
      const uint32_t vw[4] = {v0.x, v0.y, v1.x, v1.y};
      uint8_t *dst = a.vc + (((size_t)page * a.hkv + h) * a.d + d0) * kPage + off;
#pragma unroll
      for (int j = 0; j < 16; ++j) dst[j * kPage] = (uint8_t)(vw[j >> 2] >> (8 * (j & 3)));
    }
  }
}

}  // namespace

hipError_t launch_store_e4m3(const StoreE4M3Launch &a, hipStream_t s) {
  const int64_t blocks = (a.num_tokens + kPage - 1) / kPage;
  const size_t img = (size_t)a.hkv * a.d * kPage;   // one V page image
  const int use_lds = 2 * img <= 64 * 1024;
  hipLaunchKernelGGL(store_e4m3_kernel, dim3((unsigned)blocks), dim3(kStoreThreads),
                     use_lds ? 2 * img : 0, s, a, use_lds);
  return hipGetLastError();
}

}  // namespace kvq
