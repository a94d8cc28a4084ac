// NVFP4 MLA chunked prefill over the 368-byte records.
//
// local-inference-lab/vllm PR 189, "mla: wire dynamic per-token NVFP4 scaling
// and cache ABI" ("Why", "Validation"): the readers, decode and the multitile
// prefill alike, take each key's outer scale s2 from bytes [292, 296) of its
// record. New query row i of a sequence with Lq new tokens and L stored keys
// sits at position L - Lq + i and attends keys 0 .. that position with the
// decode's arithmetic:
//   s_j = softmax_scale * (s2_j * (q_lat . Kt_j) + rope_scale * (q_rope . r_j))
//   out = sum_j p_j s2_j Kt_j / sum_j p_j,   Kt_j = e2m1 * e4m3(group scale).
//
// Kernel design (gfx950, wave64): one workgroup per 8 consecutive new tokens
// of a sequence (8 waves, two per SIMD; 16 heads x 8 tokens = 128 query rows
// share every key). A step covers two pages (32 keys), so that PV runs on the
// full-rate v_mfma_f32_16x16x32_f16 with K = 32 keys.
//  * Record bytes go straight from raw buffer loads (issued before the PV
//    that precedes their use) into registers and are dequantized once per workgroup into an fp16 image of
//    the step's two pages (16 keys x 576 dims each; rows placed so that both
//    the row-slice reads of QK^T and the transposed reads of PV cover the 64
//    banks once): the latent as e2m1 * group scale (exact in fp16), the RoPE
//    part as its e4m3 value; keys past the sequence end read as zeros (the
//    buffer resource of a page covers its valid keys only).
//  * Wave w owns token w of the tile: QK^T over all 576 dims for its 16 heads
//    (A = the image rows, B = fp16 Q*2^k in registers) and its softmax. The
//    two waves of a pair (tokens 2p, 2p+1) split PV by dims (256 each) for
//    both tokens: the owner hands its fp16 P and the per-head exponent shift
//    of its running max to the partner through LDS.
//  * The softmax is the decode's: an integer-valued lazy running max (slack
//    8, log2 units) per head and the largest outer-scale exponent G of the
//    keys seen, so P = 2^(x - m) s2 2^-G <= 2^8 fits fp16 and every rescale
//    is a power of two. G depends on the keys only, so every wave computes
//    the same G sequence and rescales its own accumulators.
//  * One barrier per step. Between barriers k and k+1: the loads of step
//    k+2, PV of step k, the dequant of step k+2, QK^T and softmax of step
//    k+1. Three image buffers keep the dequant clear of the readers of
//    steps k and k+1.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kTok = 8;                    // new tokens per workgroup
constexpr int kWaves = kTok;
constexpr int kThreads = 64 * kWaves;
constexpr int kRec = 368;
constexpr int kLat = 512;
constexpr int kDqk = 576;
constexpr int kHeads = 16;
// Page image rows: key r's 576 fp16 at byte 1,184 r, a stride of 296 dwords
// (an odd multiple of 8 banks): keys r and r+8 land on the same banks. The
// gfx950 LDS serves a ds_read_b128 eight lanes at a time, lanes 8b .. 8b+7
// in the same cycle as lanes 8(b^3) .. +7; for the QK^T row-slice read
// (lane = key row + 16 * dim group) the paired blocks then hold keys 0..7
// and 8..15 four banks apart, and every cycle covers 64 distinct banks. The
// transposed PV read (8 keys x 8 dwords per pass) covers them once as well.
// Both measured conflict-free with the LDS bank-conflict counters.
constexpr int kImgRow = 2 * kDqk + 32;
constexpr int kImgBytes = 15 * kImgRow + 2 * kDqk;   // through key 15's last dim
__device__ __forceinline__ int img_row(int r) { return r * kImgRow; }
constexpr int kPageBytes = 16 * kRec;
constexpr float kTau = 8.0f;
constexpr int kGUnset = -(1 << 20);
// Q operand slices (32 dims each) kept in registers; the rest (the last
// latent slice and the RoPE part) sit in LDS, one 1 KB slab per wave
constexpr int kQReg = 14;
constexpr int kQLds = 18 - kQReg;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

struct __align__(16) PrefillMlaSmem {
  v4u xp[2][kWaves][64];          // owner's fp16 P (B-operand layout), by step parity
  uint4 sq[kQLds][kWaves][64];    // Q operand slices kQReg .. 17 of each wave's token
  int16_t xs[2][kWaves][16];      // owner's per-head exponent shift of that step
  float s2[3][32];                // the step's outer scales (0 past the sequence)
  uint8_t img[3][2][kImgBytes];   // fp16 images of a step's two pages
};

__device__ __forceinline__ uint32_t h2_bits(v2h x) { return __builtin_bit_cast(uint32_t, x); }

// Cross-lane combines without LDS or lane-index registers: the permlane swaps
// pair lane l with lane l ^ 16 (l ^ 32), the DPP moves stay within a row of
// 16 lanes (quad xor 1, quad xor 2, half-row mirror, row mirror).
__device__ __forceinline__ uint2 swap16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ uint2 swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ float max16(float v) {
  const uint2 r = swap16(__float_as_uint(v));
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float max32(float v) {
  const uint2 r = swap32(__float_as_uint(v));
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float sum16(float v) {
  const uint2 r = swap16(__float_as_uint(v));
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}
__device__ __forceinline__ float sum32(float v) {
  const uint2 r = swap32(__float_as_uint(v));
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}
__device__ __forceinline__ int imax_row16(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));    // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));    // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));   // row_half_mirror
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));   // row_mirror
  return v;
}

// Block i of n -> (sequence, tile). Blocks are dealt to the 8 XCDs round
// robin; when n is a multiple of 8, XCD x takes the consecutive tiles
// n/8 * x .. +n/8, so the workgroups that share an XCD's L2 mostly read the
// same sequence's pages at the same time.
__device__ __forceinline__ void tile_of(int i, int n, int tiles, int &b, int &t) {
  const int j = (n & 7) == 0 ? (i & 7) * (n >> 3) + (i >> 3) : i;
  b = j / tiles;
  t = j - b * tiles;
}

// The record bytes one thread dequantizes: two 16-dim groups of one key's
// latent (8 bytes of e2m1 codes and the group scale each) and 8 RoPE codes or
// the outer scale.
struct Raw {
  uint2 nib0, nib1;
  uint32_t sc0, sc1;
  uint2 rp;
};

// LDS byte addresses. An address made opaque once per step keeps the compiler
// from holding every (base + constant) of an unrolled loop in its own
// register: the constants then ride in the instructions' offset fields, and
// the transposed reads, whose builtin takes no offset, add theirs in place.
typedef __attribute__((address_space(3))) uint8_t lds_t;
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_t *)p; }
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ v4u lds_ld(uint32_t a) { return *(const __attribute__((address_space(3))) v4u *)(uintptr_t)a; }
__device__ __forceinline__ void lds_st(uint32_t a, v4u v) { *(__attribute__((address_space(3))) v4u *)(uintptr_t)a = v; }

template <int kN>
__device__ __forceinline__ void scale_all(v4f (&o)[kN], float f) {
#pragma unroll
  for (int q = 0; q < kN; ++q) o[q] *= f;
}

__global__ __launch_bounds__(kThreads) void mla_prefill_kernel(DecodeMlaLaunch a) {
  __shared__ PrefillMlaSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1;
  const int half = wave & 1;           // PV dims 256*half .. +256 of tokens 2*pair, 2*pair+1
  const int partner = wave ^ 1;
  const int row = lane & 15;
  const int grp = lane >> 4;

  const int tiles = (a.max_q_len + kTok - 1) / kTok;
  int b, tile;
  tile_of(blockIdx.x, gridDim.x, tiles, b, tile);
  const int r0 = tile * kTok;
  const int q0 = a.cu_q_lens[b];
  const int lq = a.cu_q_lens[b + 1] - q0;
  if (r0 >= lq) return;                                  // the whole workgroup
  const int L = a.seq_lens[b];
  const bool own_ok = r0 + wave < lq;
  const int pos = L - lq + r0 + wave;                    // own token's position (< 0: no key)
  const int pos_max = L - lq + min(lq, r0 + kTok) - 1;   // the tile's last token
  const int npages = pos_max >= 0 ? (pos_max >> 4) + 1 : 0;
  const int nsteps = (npages + 1) >> 1;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;

  // ---- record bytes: the waves 4*dj .. 4*dj+3 dequantize page dj of a step;
  // lane (grp, row) takes key 4*(wave&3) + grp, latent groups row and 16+row
  // (dims 16*row .. +16 and 256 + 16*row .. +16) and, for row < 8, RoPE dims
  // 8*row .. +8 (row 8: the outer scale). Its image writes then sit 32 bytes
  // apart across the lanes, which the LDS serves without bank conflicts.
  const int dj = wave >> 2;
  const int dkey = 4 * (wave & 3) + grp;
  const uint32_t off_nib = dkey * kRec + 8 * row;
  const uint32_t off_sc = dkey * kRec + 256 + row;
  const uint32_t off_rp = dkey * kRec + (row < 8 ? 304 + 8 * row : 288);
  auto fetch = [&](int s, Raw &r) {
    const int p = 2 * s + dj;
    const int nvalid = p < npages ? min(L - 16 * p, 16) : 0;
    // the page id through readfirstlane: the resource must sit in scalar registers
    const int page = nvalid > 0 ? __builtin_amdgcn_readfirstlane(bt[p]) : 0;
    const uint8_t *base = a.records + (size_t)page * kPageBytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, max(nvalid, 0) * kRec, 0x00020000);
    r.nib0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off_nib, 0, 0));
    r.nib1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off_nib + 128, 0, 0));
    r.sc0 = __builtin_amdgcn_raw_buffer_load_b8(rs, off_sc, 0, 0);
    r.sc1 = __builtin_amdgcn_raw_buffer_load_b8(rs, off_sc + 16, 0, 0);
    r.rp = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off_rp, 0, 0));
  };
  auto dequant = [&](int s, const Raw &r) {
    const uint32_t img = opaque(lds_addr(sm.img[s % 3][dj]) + img_row(dkey) + 32 * row);
    const v2h sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sc0 | (r.sc1 << 8), 1.0f, false);
    const uint32_t w[4] = {r.nib0.x, r.nib0.y, r.nib1.x, r.nib1.y};
    constexpr int kChunkOff[4] = {0, 16, 512, 528};   // dims 16*row + 0, +8, 256 + 16*row + 0, +8
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2h si = i < 2 ? v2h{sc[0], sc[0]} : v2h{sc[1], sc[1]};
      const uint4 x = make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0) * si),
                                 h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1) * si),
                                 h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2) * si),
                                 h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3) * si));
      lds_st(img + kChunkOff[i], __builtin_bit_cast(v4u, x));
    }
    if (row < 8) {
      const uint4 x = make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.rp.x, 1.0f, false)),
                                 h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.rp.x, 1.0f, true)),
                                 h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.rp.y, 1.0f, false)),
                                 h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.rp.y, 1.0f, true)));
      lds_st(img + 2 * kLat - 16 * row, __builtin_bit_cast(v4u, x));
    } else if (row == 8) {
      sm.s2[s % 3][16 * dj + dkey] = __uint_as_float(r.rp.y);
    }
  };

  Raw ra, rb;
  if (nsteps > 0) fetch(0, ra);
  if (nsteps > 1) fetch(1, rb);

  // ---- Q of the own token: each head's power of two k from all 576 dims
  // (its largest element times 2^k in [2^13, 2^14)); lane (grp, row) keeps
  // head `row`, dims 32c + 8*grp .. +8 (c < 18) as fp16 Q * 2^k
  uint4 qop[kQReg];
  int kexp = 0;
  {
    const uint4 *qp = (const uint4 *)(a.q + ((size_t)(q0 + r0 + wave) * a.hq + row) * kDqk + 8 * grp);
    uint4 qv[18];
#pragma unroll
    for (int c = 0; c < 18; ++c) qv[c] = own_ok ? qp[4 * c] : make_uint4(0, 0, 0, 0);
    uint32_t am = 0;
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      const uint32_t w[4] = {qv[c].x, qv[c].y, qv[c].z, qv[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
    {
      const uint2 r = swap16(am);
      am = max(r.x, r.y);
    }
    {
      const uint2 r = swap32(am);
      am = max(r.x, r.y);
    }
    kexp = am == 0 ? 0 : 14 - __builtin_amdgcn_frexp_expf(__uint_as_float(am << 16));
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      const uint32_t w[4] = {qv[c].x, qv[c].y, qv[c].z, qv[c].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = h2_bits(v2h{(_Float16)__builtin_ldexpf(bf16lo(w[i]), kexp), (_Float16)__builtin_ldexpf(bf16hi(w[i]), kexp)});
      const uint4 v = make_uint4(o[0], o[1], o[2], o[3]);
      if (c < kQReg) qop[c] = v;
      else sm.sq[c - kQReg][wave][lane] = v;
    }
  }
  const float c_score = __builtin_ldexpf(a.scale_log2, -kexp);
  const float c_rope = a.rope_scale * c_score;

  float m_run = -INFINITY;
  float l_run = 0.0f;
  int Gs = kGUnset;
  v4f o0[16], o1[16];                  // PV accumulators of tokens 2*pair and 2*pair+1
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    o0[t] = v4f{0.f, 0.f, 0.f, 0.f};
    o1[t] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  v4u po = v4u{0u, 0u, 0u, 0u};        // own P of the step in flight

  // QK^T A operand: key `row`, dims 32c + 8*grp; PV A operand (transposed):
  // lane s of group grp reads key 4*grp + s/4, dims 256*half + 16q + 4(s%4)
  const int a_off = img_row(row) + 16 * grp;
  const int t_off = img_row(4 * grp + (row >> 2)) + 2 * (256 * half + 4 * (row & 3));

  // ---- QK^T and softmax of step s for the own token; P to LDS for the partner
  auto qk_softmax = [&](int s) {
    const uint32_t i0 = opaque(lds_addr(sm.img[s % 3][0]) + a_off);
    const uint32_t qs = opaque(lds_addr(&sm.sq[0][wave][lane]));
    const float *s2t = sm.s2[s % 3];
    // the outer-scale exponent: the same for every wave
    {
      const float sa = s2t[row];
      const float sb = s2t[16 + row];
      int e = max(sa > 0.0f ? __builtin_amdgcn_frexp_expf(sa) : kGUnset,
                  sb > 0.0f ? __builtin_amdgcn_frexp_expf(sb) : kGUnset);
      if (__ballot(e > Gs)) {
        e = imax_row16(e);
        const int g_new = __builtin_amdgcn_readfirstlane(e);
        if (Gs != kGUnset) {
          const float f = __builtin_ldexpf(1.0f, max(Gs - g_new, -200));
          scale_all(o0, f);
          scale_all(o1, f);
        }
        Gs = g_new;
      }
    }
    int sh = 0;
    v4u pw = v4u{0u, 0u, 0u, 0u};
    if (own_ok && 32 * s <= pos) {
      v4f al0 = v4f{0.f, 0.f, 0.f, 0.f}, al1 = al0, ar0 = al0, ar1 = al0;
      // software pipelined like PV: the operands of slice c+1 are requested
      // before the multiplies of slice c
      struct Op {
        v4u x0, x1;
        uint4 qb;
      };
      auto rdk = [&](int c) {
        Op r;
        r.x0 = lds_ld(i0 + 64 * c);
        r.x1 = lds_ld(i0 + kImgBytes + 64 * c);
        r.qb = c < kQReg ? qop[c < kQReg ? c : 0] : __builtin_bit_cast(uint4, lds_ld(qs + (c < kQReg ? 0 : c - kQReg) * kWaves * 1024));
        return r;
      };
      Op nx = rdk(0);
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        const Op cu = nx;
        if (c + 1 < 18) nx = rdk(c + 1);
        const v8h qb = __builtin_bit_cast(v8h, cu.qb);
        if (c < 16) {
          al0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, cu.x0), qb, al0, 0, 0, 0);
          al1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, cu.x1), qb, al1, 0, 0, 0);
        } else {
          ar0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, cu.x0), qb, ar0, 0, 0, 0);
          ar1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, cu.x1), qb, ar1, 0, 0, 0);
        }
      }
      // order: the operand reads run one multiply ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
      for (int c = 0; c + 1 < kQReg; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
#pragma unroll
      for (int c = kQReg - 1; c < 17; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      // keys 4*grp + i of page j: scores in log2 units
      const v4f sk0 = *(const v4f *)(s2t + 4 * grp);
      const v4f sk1 = *(const v4f *)(s2t + 16 + 4 * grp);
      float x[8], s2k[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s2k[i] = sk0[i];
        s2k[4 + i] = sk1[i];
        x[i] = fmaf(c_score * sk0[i], al0[i], c_rope * ar0[i]);
        x[4 + i] = fmaf(c_score * sk1[i], al1[i], c_rope * ar1[i]);
      }
      if (32 * s + 31 > pos) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (32 * s + 16 * (i >> 2) + 4 * grp + (i & 3) > pos) x[i] = -INFINITY;
      }
      bool raise_m = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) raise_m |= x[i] > m_run + kTau;
      if (__ballot(raise_m)) {
        float bmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        bmax = max32(max16(bmax));
        if (bmax > m_run + kTau) {
          const float m_new = __builtin_ceilf(bmax);
          sh = m_run == -INFINITY ? -1000 : (int)(m_run - m_new);
          const float alpha = __builtin_ldexpf(1.0f, max(sh, -200));
          l_run *= alpha;
          if (half == 0) scale_all(o0, alpha);
          else scale_all(o1, alpha);
          m_run = m_new;
        }
      }
      const float g = __builtin_ldexpf(1.0f, -Gs);   // s2 * g < 1
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pe = __builtin_amdgcn_exp2f(x[i] - m_run);   // <= 2^8
        l_run += pe;
        pv[i] = pe * (s2k[i] * g);
      }
      pw = v4u{h2_bits(v2h{(_Float16)pv[0], (_Float16)pv[1]}), h2_bits(v2h{(_Float16)pv[2], (_Float16)pv[3]}),
               h2_bits(v2h{(_Float16)pv[4], (_Float16)pv[5]}), h2_bits(v2h{(_Float16)pv[6], (_Float16)pv[7]})};
    }
    po = pw;
    sm.xp[s & 1][wave][lane] = pw;
    if (lane < 16) sm.xs[s & 1][wave][lane] = (int16_t)max(sh, -200);
  };

  // ---- PV of step s for both tokens of the pair on dims 256*half .. +256
  auto pv_step = [&](int s) {
    const v4u pp = sm.xp[s & 1][partner][lane];
    const int shp = sm.xs[s & 1][partner][row];
    if (__ballot(shp != 0)) {
      const float f = __builtin_ldexpf(1.0f, max(shp, -200));
      if (half == 0) scale_all(o1, f);
      else scale_all(o0, f);
    }
    const v8h pb0 = __builtin_bit_cast(v8h, half == 0 ? po : pp);
    const v8h pb1 = __builtin_bit_cast(v8h, half == 0 ? pp : po);
    uint32_t v0 = opaque(lds_addr(sm.img[s % 3][0]) + t_off);
    // software pipelined: the operand of tile q+1 is requested before the
    // multiplies of tile q
    auto rd = [&]() {
      const v4s va0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(uintptr_t)v0);
      const v4s va1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(uintptr_t)(v0 + kImgBytes));
      v0 = opaque(v0 + 32);
      return __builtin_bit_cast(v8h, __builtin_shufflevector(va0, va1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    v8h va_n = rd();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const v8h va = va_n;
      if (q + 1 < 16) va_n = rd();
      o0[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb0, o0[q], 0, 0, 0);
      o1[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb1, o1[q], 0, 0, 0);
    }
    // keep that order through scheduling: reads of tile q+1, then the two
    // multiplies of tile q
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int q = 0; q < 15; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  // prologue: steps 0 and 1 dequantized, softmax of step 0
  if (nsteps > 0) {
    dequant(0, ra);
    if (nsteps > 1) dequant(1, rb);
    __syncthreads();
    qk_softmax(0);
    __syncthreads();
  }
  for (int k = 0; k < nsteps; ++k) {
    // the record bytes of step k+2 are requested before PV of step k and
    // dequantized after it (not held in registers through QK^T and softmax)
    if (k + 2 < nsteps) fetch(k + 2, ra);
    // PV at the highest wave priority: the other wave of the SIMD fills the
    // matrix unit's busy cycles with its vector work
    __builtin_amdgcn_s_setprio(2);
    pv_step(k);
    __builtin_amdgcn_s_setprio(0);
    if (k + 2 < nsteps) dequant(k + 2, ra);
    if (k + 1 < nsteps) {
      qk_softmax(k + 1);
      __syncthreads();
    }
  }

  // ---- out = 2^G O / l (zeros when no key contributed); the row sums of both
  // tokens come from their owners
  l_run = sum32(sum16(l_run));
  // the lane index again from the hardware counter (cheaper than keeping it
  // in a register across the loop)
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int row_e = lane_e & 15;
  const int grp_e = lane_e >> 4;
  // the row sums go where the P exchange was, once every wave is past its
  // last PV
  float *fin = (float *)&sm.xp[0][0][0];
  __syncthreads();
  if (lane_e < 16) fin[16 * wave + lane_e] = l_run;
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = 2 * pair + t;
    if (r0 + tok >= lq) continue;
    const float l = fin[16 * tok + row_e];
    float sc = 0.0f;
    if (l > 0.0f && Gs != kGUnset) sc = __builtin_ldexpf(1.0f / l, Gs);
    uint16_t *dst = a.out + ((size_t)(q0 + r0 + tok) * a.hq + row_e) * kLat + 256 * half + 4 * grp_e;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const v4f v = t == 0 ? o0[q] : o1[q];
      uint2 w;
      w.x = f32_to_bf16_bits(v[0] * sc) | (f32_to_bf16_bits(v[1] * sc) << 16);
      w.y = f32_to_bf16_bits(v[2] * sc) | (f32_to_bf16_bits(v[3] * sc) << 16);
      *(uint2 *)(dst + 16 * q) = w;
    }
  }
}

}  // namespace

hipError_t launch_prefill_mla(const DecodeMlaLaunch &a, int max_seq_len, hipStream_t s) {
  (void)max_seq_len;
  if (a.hq != kHeads || a.cu_q_lens == nullptr || a.max_q_len <= 0) return hipErrorInvalidValue;
  const size_t tiles = (size_t)(a.max_q_len + kTok - 1) / kTok;
  hipLaunchKernelGGL(mla_prefill_kernel, dim3((unsigned)((size_t)a.batch * tiles)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
