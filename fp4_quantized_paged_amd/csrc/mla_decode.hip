// NVFP4 MLA decode: attention of 16 query heads over one latent KV head
// stored as 368-byte NVFP4 records.
//
// local-inference-lab/vllm PR 189, "mla: wire dynamic per-token NVFP4 scaling
// and cache ABI" (commit message, "Why"): readers take the per-token outer
// scale from bytes [292, 296) of each record instead of a per-layer launch
// scalar. Per key j:
//   latent_j = e2m1(v) * e4m3(sg) * s2_j        (the group product is exact in bf16)
//   K_j = [latent_j ; e4m3(rope_j) * rope_scale],  V_j = latent_j
//   s_j = softmax_scale * (s2_j * (q_lat . Kt_j) + rope_scale * (q_rope . r_j))
// with Kt_j = e2m1 * e4m3(sg); out = sum_j p_j s2_j Kt_j / sum_j p_j.
//
// Kernel design (gfx950, wave64, 8 waves per workgroup, one workgroup per
// (sequence, split), waves take interleaved 16-token pages; Q sits in LDS):
//  * QK^T on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 latent dims, B = the
//    16 query heads. Lane (key l%16, group g) dequantizes dims 128g + 8c..+8
//    for step c straight from its record (hardware fp4 -> fp32 conversion at
//    unit scale, then the fp32 group scale, packed to bf16) and feeds the MFMA
//    from registers; the RoPE part takes two more MFMAs with its own
//    accumulator;
//  * the same bf16 values go to LDS row-major ([key][dim], rows padded to
//    avoid bank conflicts); PV (v_mfma_f32_16x16x16_bf16, A = V^T) reads them
//    back with ds_read_b64_tr_b16, whose 16-lane transpose turns four row
//    segments into one dim x 4 keys operand: no transposed copy is written;
//  * the S^T output lane (keys 4g..4g+3 of head l%16) is already the B
//    operand of the 16x16x16 PV step; s2 is folded into P;
//  * waves merge through LDS; with one split the workgroup writes bf16, else
//    partials go to the workspace for the shared split combine.
#include "kvq_combine.h"
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kMW = 8;                // waves per workgroup (one workgroup per CU)
constexpr int kRec = 368;
constexpr int kLat = 512;
constexpr int kRowB = 2 * kLat + 32;  // LDS bytes per key row (pad: conflict-free transpose reads)
constexpr int kHeads = 16;
constexpr int kQRowB = 2 * (kLat + 64) + 16;   // LDS bytes per query head (pad: conflict-free)

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8bf as_v8bf(uint4 x) { return __builtin_bit_cast(v8bf, x); }

__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  // both values are exactly representable in bf16: keep the upper halves
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 e2m1 codes (one dword, element 2i in the low nibble of byte i) times the
// group scale, as 8 exact bf16
template <int kB>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t w, float sg) {
  const v2f f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, kB);
  return pack_bf16_exact(f.x * sg, f.y * sg);
}
__device__ __forceinline__ uint4 dequant8(uint32_t w, float sg) {
  return make_uint4(fp4_pair_bf16<0>(w, sg), fp4_pair_bf16<1>(w, sg), fp4_pair_bf16<2>(w, sg),
                    fp4_pair_bf16<3>(w, sg));
}

// 8 e4m3 codes (two dwords) as 8 exact bf16
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3_pair_bf16(uint32_t w) {
  const v2f f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
  return pack_bf16_exact(f.x, f.y);
}
__device__ __forceinline__ uint4 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  return make_uint4(e4m3_pair_bf16<false>(w0), e4m3_pair_bf16<true>(w0), e4m3_pair_bf16<false>(w1),
                    e4m3_pair_bf16<true>(w1));
}

__device__ __forceinline__ float e4m3_byte(uint32_t w, int byte) {
  const v2f f = __builtin_amdgcn_cvt_pk_f32_fp8((int)((w >> (8 * byte)) & 0xFFu), false);
  return f.x;
}

__global__ __launch_bounds__(64 * kMW) __attribute__((amdgpu_waves_per_eu(2)))
void mla_decode_kernel(DecodeMlaLaunch a, int splits, int pages_per_split) {
  __shared__ __align__(16) uint8_t smem[kMW * kHeads * kRowB];
  __shared__ __align__(16) uint8_t qs[kHeads * kQRowB];   // Q, bf16 [head][576]
  __shared__ float s_m[kMW][kHeads], s_l[kMW][kHeads];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;      // key of the A operand / head of the output
  const int grp = lane >> 4;
  const int b = blockIdx.x / splits;
  const int split = blockIdx.x - b * splits;

  const int L = a.seq_lens[b];
  const int npages = (L + 15) >> 4;
  const int p_begin = split * pages_per_split;
  const int p_end = min(npages, p_begin + pages_per_split);

  // ---- Q (16 heads x 576 bf16) into LDS; the Q^T operand of head `row` for
  // latent step c covers dims 128*grp + 8c, RoPE step r dims 512 + 16*grp + 8r
  {
    const uint4 *qsrc = (const uint4 *)(a.q + (size_t)b * a.hq * (kLat + 64));
    for (int c = threadIdx.x; c < kHeads * (kLat + 64) / 8; c += 64 * kMW) {
      const int h = c / ((kLat + 64) / 8);
      const int part = c - h * ((kLat + 64) / 8);
      *(uint4 *)(qs + h * kQRowB + 16 * part) = qsrc[c];
    }
  }
  __syncthreads();
  const uint8_t *qrow = qs + row * kQRowB;

  float m_run = -INFINITY;
  float l_run = 0.0f;
  v4f o[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};

  uint8_t *kt = smem + wave * kHeads * kRowB;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;

  for (int p = p_begin + wave; p < p_end; p += kMW) {
    const uint8_t *rec = a.records + (size_t)bt[p] * (16 * kRec);
    const uint8_t *mine = rec + row * kRec;
    const bool key_ok = p * 16 + row < L;
    v4u nib[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) nib[i] = __builtin_nontemporal_load((const v4u *)(mine + 64 * grp + 16 * i));
    const uint2 sc = *(const uint2 *)(mine + 256 + 8 * grp);
    const v4u rp = __builtin_nontemporal_load((const v4u *)(mine + 304 + 16 * grp));

    // ---- dequant + QK^T (latent), rows also to LDS for PV
    v4f acc_lat = v4f{0.f, 0.f, 0.f, 0.f};
    uint8_t *ktrow = kt + row * kRowB + 256 * grp;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t w = nib[c >> 2][c & 3];
      const float sg = e4m3_byte((c >> 1) < 4 ? sc.x : sc.y, (c >> 1) & 3);
      uint4 x = dequant8(w, sg);
      if (!key_ok) x = make_uint4(0, 0, 0, 0);
      *(uint4 *)(ktrow + 16 * c) = x;
      const uint4 qop = *(const uint4 *)(qrow + 256 * grp + 16 * c);
      acc_lat = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(x), as_v8bf(qop), acc_lat, 0, 0, 0);
    }
    // ---- RoPE part
    v4f acc_rope = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint4 x = e4m3x8_bf16(rp[2 * r], rp[2 * r + 1]);
      if (!key_ok) x = make_uint4(0, 0, 0, 0);
      const uint4 qop = *(const uint4 *)(qrow + 2 * kLat + 32 * grp + 16 * r);
      acc_rope = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(x), as_v8bf(qop), acc_rope, 0, 0, 0);
    }

    // ---- scores of keys 4*grp + i for head `row`
    float x[4], s2v[4];
    float bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * grp + i;
      const bool ok = p * 16 + k < L;
      s2v[i] = ok ? *(const float *)(rec + k * kRec + 292) : 0.0f;
      x[i] = ok ? a.scale_log2 * fmaf(s2v[i], acc_lat[i], a.rope_scale * acc_rope[i]) : -INFINITY;
      bmax = fmaxf(bmax, x[i]);
    }
    bmax = wave_max_xor(bmax, 16);
    bmax = wave_max_xor(bmax, 32);
    const float m_new = fmaxf(m_run, bmax);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float pw[4], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = __builtin_amdgcn_exp2f(x[i] - m_use);
      psum += pe;
      pw[i] = pe * s2v[i];
    }
    l_run = l_run * alpha + psum;
    typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
    const v4bf pb4 = {(__bf16)pw[0], (__bf16)pw[1], (__bf16)pw[2], (__bf16)pw[3]};
    const v4s pb = __builtin_bit_cast(v4s, pb4);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < 32; ++t) o[t] *= alpha;
    }

    // ---- PV: lane s of each 16-lane group fetches 8 bytes of key row
    // 4*grp + s/4 at dims 16t + 4*(s%4); the transpose read hands lane j the
    // dim 16t + j of keys 4*grp .. 4*grp+3
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint8_t *trbase = kt + (4 * grp + (row >> 2)) * kRowB + 8 * (row & 3);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const v4s va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s *)(trbase + 32 * t));
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[t], 0, 0, 0);
      // bound the transpose reads in flight (each holds two registers)
      if ((t & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the waves (lane holds O[head row][dims 16t + 4*grp + i])
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (grp == 0) {
    s_m[wave][row] = m_run;
    s_l[wave][row] = l_run;
  }
  __syncthreads();
  {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMW; ++w) M = fmaxf(M, s_m[w][row]);
    const float f = __builtin_amdgcn_exp2f(m_run - (M == -INFINITY ? 0.0f : M));
#pragma unroll
    for (int t = 0; t < 32; ++t) o[t] *= f;
  }
  float *slab = (float *)smem;          // [kMW/2][16 heads][512 dims]
  constexpr int H = kMW / 2;
  if (wave >= H) {
#pragma unroll
    for (int t = 0; t < 32; ++t)
      *(v4f *)(slab + ((size_t)(wave - H) * kHeads + row) * kLat + 16 * t + 4 * grp) = o[t];
  }
  __syncthreads();
  if (wave < H) {
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      float *dst = slab + ((size_t)wave * kHeads + row) * kLat + 16 * t + 4 * grp;
      *(v4f *)dst = o[t] + *(const v4f *)dst;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kHeads * kLat; e += 64 * kMW) {
    const int h = e / kLat;
    const int d = e - h * kLat;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMW; ++w) M = fmaxf(M, s_m[w][h]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kMW; ++w) den += __builtin_amdgcn_exp2f(s_m[w][h] - Mu) * s_l[w][h];
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < H; ++w) acc += slab[((size_t)w * kHeads + h) * kLat + d];
    if (splits == 1) {
      const float val = den > 0.0f ? acc / den : 0.0f;
      a.out[((size_t)b * a.hq + h) * kLat + d] = (uint16_t)f32_to_bf16_bits(val);
    } else {
      const size_t pi = ((size_t)b * a.hq + h) * splits + split;
      a.part_o[pi * kLat + d] = acc;
      if (d == 0) {
        a.part_ml[2 * pi] = M;
        a.part_ml[2 * pi + 1] = den;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_mla(const DecodeMlaLaunch &a, const MlaPlan &p, hipStream_t s) {
  if (a.hq != kHeads) return hipErrorNotSupported;
  hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)((size_t)a.batch * p.splits)), dim3(64 * kMW), 0, s, a,
                     p.splits, p.pages_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL((split_combine_kernel<kLat>), dim3((unsigned)((size_t)a.batch * a.hq)), dim3(kLat), 0, s,
                     a.part_o, a.part_ml, a.out, p.splits, 1.0f);
  return hipGetLastError();
}

}  // namespace kvq
