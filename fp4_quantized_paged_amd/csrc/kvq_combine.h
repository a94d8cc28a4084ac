// Split-KV combine shared by the decode kernels: merges per-split online-
// softmax partials (o unnormalised, m in the log2 domain, l) of each
// (sequence, query head) into the bf16 output:
//   out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Splits that saw no key carry m = -inf and l = 0 and drop out; a row with no
// key at all outputs zeros.
#pragma once

#include "kvq_device.h"

namespace kvq {

template <int D>
__global__ __launch_bounds__(D) void split_combine_kernel(const float *part_o, const float *part_ml,
                                                          uint16_t *out, int splits, float v_scale) {
  // Up to kPre splits: every partial is requested before any is used (one
  // memory round trip); more splits take the plain loops. Both orders of
  // operations are the same: the max first, then the sums in split order.
  constexpr int kPre = 16;
  const int bh = blockIdx.x;          // b * hq + h
  const int dcol = threadIdx.x;
  const float *ml = part_ml + (size_t)bh * splits * 2;
  const float *po = part_o + (size_t)bh * splits * D + dcol;
  float acc = 0.0f, den = 0.0f;
  if (splits <= kPre) {
    float mv[kPre], lv[kPre], ov[kPre];
#pragma unroll
    for (int s = 0; s < kPre; ++s) {
      const int c = min(s, splits - 1);   // clamped copies past the last split are not used
      mv[s] = ml[2 * c];
      lv[s] = ml[2 * c + 1];
      ov[s] = po[(size_t)c * D];
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kPre; ++s)
      if (s < splits) M = fmaxf(M, mv[s]);
    const float Mu = M == -INFINITY ? 0.0f : M;
#pragma unroll
    for (int s = 0; s < kPre; ++s) {
      if (s < splits) {
        const float f = __builtin_amdgcn_exp2f(mv[s] - Mu);
        acc += f * ov[s];
        den += f * lv[s];
      }
    }
  } else {
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    for (int s = 0; s < splits; ++s) {
      const float f = __builtin_amdgcn_exp2f(ml[2 * s] - Mu);
      acc += f * po[(size_t)s * D];
      den += f * ml[2 * s + 1];
    }
  }
  const float val = den > 0.0f ? (acc / den) * v_scale : 0.0f;
  out[(size_t)bh * D + dcol] = (uint16_t)f32_to_bf16_bits(val);
}

}  // namespace kvq
