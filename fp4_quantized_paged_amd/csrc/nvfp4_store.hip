// NVFP4 368-byte MLA latent record store.
//
// local-inference-lab/vllm PR 189, "mla: wire dynamic per-token NVFP4 scaling
// and cache ABI" (commit message, "Why"): the 512-dim latent is stored as e2m1
// values with one E4M3 scale per group, next to an fp8 RoPE part, and the
// writer derives a per-token second-level scale that it stores inside the
// record at bytes [292, 296) of existing padding; the record stays 368 bytes.
//
// Per token (all arithmetic fp32, divisions correctly rounded):
//   s2 = amax(latent) / 2688                  (2688 = e2m1 max 6 * e4m3 max 448)
//   group g (16 elements): sg = e4m3_RNE(min(ag / fp32(6 * s2), 448))
//   dg = fp32(e4m3(sg) * s2); codes = e2m1_RNE(clip(x * fp32(1 / dg), -6, 6)),
//   or +0 codes when dg == 0 (also for an all-zero token, where s2 = 0)
//   RoPE: the e4m3 store quantizer with the rope scale
// Static mode (the writer the same commit message describes before the
// per-token scale: one outer scale per layer, 1.0 unless calibrated): s2 is
// that launch constant for every token, with the same formulas; a group whose
// ratio ag / (6 s2) falls below 2^-6 gets a subnormal or zero scale code.
// Record: [0,256) values, element 2i in the low nibble of byte i; [256,288)
// group-scale codes; [288,292) zero; [292,296) s2 (little endian);
// [296,304) zero; [304,368) RoPE codes.
//
// One 32-lane half of a wave handles one token per pass, one lane per
// 16-element group (plus two RoPE elements per lane); the loads of every pass
// are issued before any token is encoded. The records are assembled in LDS
// and leave as 23 16-byte stores each, with the slots kept in LDS; the records
// of a workgroup (half a page in a bulk store) are contiguous.
#include "kvq_device.h"
#include "kvq_launch.h"

#pragma clang fp contract(off)

namespace kvq {

namespace {

constexpr int kRec = 368;
constexpr int kThreads = 256;
constexpr int kHalves = kThreads / 32;    // half waves: one token each per pass
constexpr int kPasses = 1;                // tokens per half wave (2: same bulk rate, slower short stores; 4: slower)
constexpr int kTokensPerBlock = kHalves * kPasses;

// Eight values (the four bf16 pairs of w) times r as e2m1 codes, element 2i
// in the low nibble of byte i: clipped to [-6, 6] (med3 keeps the sign of a
// zero), then the gfx950 fp4 conversion with a unit scale, which rounds to the
// nearest code, ties to the even one, and keeps the sign bit (the same result
// as rint on the magnitude scaled per binade: the grid is evenly spaced inside
// each binade).
__device__ __forceinline__ float clip6(float y) { return __builtin_amdgcn_fmed3f(y, -6.0f, 6.0f); }

__device__ __forceinline__ uint32_t e2m1x8(const uint32_t *w, float r) {
  uint32_t p = 0u;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, clip6(bf16lo(w[0]) * r), clip6(bf16hi(w[0]) * r), 1.0f, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, clip6(bf16lo(w[1]) * r), clip6(bf16hi(w[1]) * r), 1.0f, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, clip6(bf16lo(w[2]) * r), clip6(bf16hi(w[2]) * r), 1.0f, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, clip6(bf16lo(w[3]) * r), clip6(bf16hi(w[3]) * r), 1.0f, 3);
  return p;
}

// One token's record, from its already loaded elements, into LDS.
__device__ __forceinline__ void encode_token(const StoreNvfp4Launch &a, uint4 x0, uint4 x1, uint32_t rp, int g,
                                             uint8_t *R) {
  const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};

  // ---- group amax (|bf16| orders like its bits), token amax over 32 lanes
  uint32_t ag_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ag_bits = max(ag_bits, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  uint32_t am_bits = ag_bits;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) am_bits = max(am_bits, (uint32_t)__shfl_xor((int)am_bits, off, 32));
  const float ag = __uint_as_float(ag_bits << 16);
  const float amax = __uint_as_float(am_bits << 16);

  // ---- two-level scales
  const float s2 = a.static_s2 > 0.0f ? a.static_s2 : amax / 2688.0f;
  const float d = 6.0f * s2;
  float ratio = amax > 0.0f ? ag / d : 0.0f;
  ratio = fminf(ratio, kE4M3Max);
  const uint32_t sg = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ratio, 0.0f, 0, false) & 0xFFu;
  const v2f sgpair = __builtin_amdgcn_cvt_pk_f32_fp8((int)sg, false);
  const float sgv = sgpair.x;
  const float dg = sgv * s2;
  const float r = dg != 0.0f ? 1.0f / dg : 0.0f;

  // ---- e2m1 codes, two per byte (element 2i low nibble)
  uint32_t packed[2] = {0u, 0u};
  if (dg != 0.0f) {
    packed[0] = e2m1x8(w, r);
    packed[1] = e2m1x8(w + 4, r);
  }
  // ---- RoPE pair through the e4m3 store quantizer
  const uint32_t rope = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(bf16lo(rp) * a.rope_inv),
                                                                  sat448(bf16hi(rp) * a.rope_inv), 0, false) &
                        0xFFFFu;

  // ---- the record in LDS
  *(uint2 *)(R + 8 * g) = make_uint2(packed[0], packed[1]);
  R[256 + g] = (uint8_t)sg;
  *(uint16_t *)(R + 304 + 2 * g) = (uint16_t)rope;
  if (g == 0) {
    *(uint32_t *)(R + 288) = 0u;
    *(float *)(R + 292) = s2;
    *(uint2 *)(R + 296) = make_uint2(0u, 0u);
  }
}

__global__ __launch_bounds__(kThreads) void store_nvfp4_kernel(StoreNvfp4Launch a) {
  __shared__ __align__(16) uint8_t rec[kTokensPerBlock][kRec];
  __shared__ int64_t sslot[kTokensPerBlock];   // the records' slots, for the store phase
  const int tid = threadIdx.x;
  const int half = tid >> 5;                 // token slot within a pass
  const int g = tid & 31;                    // latent group / RoPE pair
  const int64_t tb = (int64_t)blockIdx.x * kTokensPerBlock;

  // ---- every pass's loads first (the half wave's tokens half, half + 8, ...)
  uint4 x0[kPasses], x1[kPasses];
  uint32_t rp[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t t = tb + p * kHalves + half;
    const int64_t slot = t < a.num_tokens ? a.slot[t] : -1;
    if (g == 0) sslot[p * kHalves + half] = slot;
    x0[p] = x1[p] = make_uint4(0, 0, 0, 0);
    rp[p] = 0;
    if (slot >= 0) {
      const uint16_t *src = a.x + t * a.stride;
      const v4u w0 = __builtin_nontemporal_load((const v4u *)(src + 16 * g));
      const v4u w1 = __builtin_nontemporal_load((const v4u *)(src + 16 * g + 8));
      x0[p] = make_uint4(w0.x, w0.y, w0.z, w0.w);
      x1[p] = make_uint4(w1.x, w1.y, w1.z, w1.w);
      rp[p] = *(const uint32_t *)(src + 512 + 2 * g);
    }
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) encode_token(a, x0[p], x1[p], rp[p], g, rec[p * kHalves + half]);
  __syncthreads();

  // ---- 23 16-byte stores per record
  for (int c = tid; c < kTokensPerBlock * (kRec / 16); c += kThreads) {
    const int tok = c / (kRec / 16);
    const int part = c - tok * (kRec / 16);
    const int64_t s = sslot[tok];   // -1 past the last token and for skipped tokens
    if (s < 0) continue;
    const v4u v = *(const v4u *)(rec[tok] + 16 * part);
    __builtin_nontemporal_store(v, (v4u *)(a.records + (size_t)s * kRec + 16 * part));
  }
}

}  // namespace

hipError_t launch_store_nvfp4(const StoreNvfp4Launch &a, hipStream_t s) {
  const int64_t blocks = (a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(store_nvfp4_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
