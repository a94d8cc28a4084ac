// Device-side helpers shared by the kvq kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPage = 16;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Saturating clamp to the e4m3 finite range; NaN passes through unchanged
// (a NaN compares false), so it converts to the NaN code.
__device__ __forceinline__ float sat448(float y) {
  return fabsf(y) > kE4M3Max ? __builtin_copysignf(kE4M3Max, y) : y;
}

// Four fp32 -> four OCP e4m3 bytes (byte i = value i), hardware RNE
// conversion (v_cvt_pk_fp8_f32; gfx950 uses the OCP e4m3fn encoding).
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// Quantize 8 bf16 (packed in a uint4) with a multiply by the reciprocal scale
// and the saturating clamp; returns 8 e4m3 bytes.
__device__ __forceinline__ uint2 quant8_e4m3(uint4 x, float inv) {
  uint2 r;
  r.x = cvt4_e4m3(sat448(bf16lo(x.x) * inv), sat448(bf16hi(x.x) * inv),
                  sat448(bf16lo(x.y) * inv), sat448(bf16hi(x.y) * inv));
  r.y = cvt4_e4m3(sat448(bf16lo(x.z) * inv), sat448(bf16hi(x.z) * inv),
                  sat448(bf16lo(x.w) * inv), sat448(bf16hi(x.w) * inv));
  return r;
}

// Round an fp32 to bf16 bits, nearest-even (finite inputs and NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// bf16 rounding of a finite fp32 value, returned as fp32.
__device__ __forceinline__ float round_bf16_finite(float f) {
  uint32_t u = __float_as_uint(f);
  return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}

// D += A * B with A: 16 x 128 and B: 128 x 16 e4m3 operands, fp32 accum.
// Lane l holds row (l % 16) of A / column (l % 16) of B and a 32-byte slice of
// K selected by l / 16; A and B use the same K ordering.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace kvq
