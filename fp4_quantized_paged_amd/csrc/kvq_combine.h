// Split-KV combine shared by the decode kernels: merges per-split online-
// softmax partials (o unnormalised, m in the log2 domain, l) of each
// (sequence, query head) into the bf16 output:
//   out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Splits that saw no key carry m = -inf and l = 0 and drop out; a row with no
// key at all outputs zeros.
#pragma once

#include "kvq_device.h"

namespace kvq {

// One workgroup per (sequence, query head): G = blockDim.x / D thread groups
// of D threads (one per dim; G from combine_groups, at most
// kCombineGroups) take consecutive ranges of the splits, so a long split
// list is read by G times the threads; each thread requests up to kCombinePre
// splits' partials before it uses any (one memory round trip for up to
// G * kCombinePre splits). Order of operations, fixed for a given split
// count: M is the max of all m_s; each group sums its range in split order;
// the group sums are added in group order.
constexpr int kCombineGroups = 8;
constexpr int kCombinePre = 16;
inline int combine_groups(int splits) {
  const int g = (splits + kCombinePre - 1) / kCombinePre;
  return g < 1 ? 1 : (g > kCombineGroups ? kCombineGroups : g);
}

template <int D>
__global__ __launch_bounds__(D * kCombineGroups) void split_combine_kernel(const float *part_o, const float *part_ml,
                                                                           uint16_t *out, int splits, float v_scale) {
  constexpr int kPre = kCombinePre;
  __shared__ float s_m[kCombineGroups];
  __shared__ float s_acc[kCombineGroups][D];
  __shared__ float s_den[kCombineGroups][D];
  const int bh = blockIdx.x;          // b * hq + h
  const int dcol = threadIdx.x % D;
  const int g = threadIdx.x / D;
  const int ng = blockDim.x / D;
  const int per = (splits + ng - 1) / ng;
  const int s0 = min(g * per, splits);
  const int s1 = min(s0 + per, splits);
  const float *ml = part_ml + (size_t)bh * splits * 2;
  const float *po = part_o + (size_t)bh * splits * D + dcol;

  // the group's max; its first kPre splits' partials are requested with it
  float mv[kPre], lv[kPre], ov[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    // clamped: copies past the range are loaded (no branch between the
    // requests) but not used
    const int c = min(s0 + i, splits - 1);
    mv[i] = ml[2 * c];
    lv[i] = ml[2 * c + 1];
    ov[i] = po[(size_t)c * D];
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPre; ++i)
    if (s0 + i < s1) M = fmaxf(M, mv[i]);
  for (int sb = s0 + kPre; sb < s1; sb += kPre) {
    float mc[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) mc[i] = ml[2 * min(sb + i, splits - 1)];
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      if (sb + i < s1) M = fmaxf(M, mc[i]);
  }
  if (dcol == 0) s_m[g] = M;
  __syncthreads();
  M = s_m[0];
  for (int i = 1; i < ng; ++i) M = fmaxf(M, s_m[i]);
  const float Mu = M == -INFINITY ? 0.0f : M;

  float acc = 0.0f, den = 0.0f;
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    if (s0 + i < s1) {
      const float f = __builtin_amdgcn_exp2f(mv[i] - Mu);
      acc += f * ov[i];
      den += f * lv[i];
    }
  }
  for (int sb = s0 + kPre; sb < s1; sb += kPre) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int c = min(sb + i, splits - 1);
      mv[i] = ml[2 * c];
      lv[i] = ml[2 * c + 1];
      ov[i] = po[(size_t)c * D];
    }
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      if (sb + i < s1) {
        const float f = __builtin_amdgcn_exp2f(mv[i] - Mu);
        acc += f * ov[i];
        den += f * lv[i];
      }
    }
  }
  s_acc[g][dcol] = acc;
  s_den[g][dcol] = den;
  __syncthreads();
  if (g == 0) {
    for (int i = 1; i < ng; ++i) {
      acc += s_acc[i][dcol];
      den += s_den[i][dcol];
    }
    const float val = den > 0.0f ? (acc / den) * v_scale : 0.0f;
    out[(size_t)bh * D + dcol] = (uint16_t)f32_to_bf16_bits(val);
  }
}

}  // namespace kvq
