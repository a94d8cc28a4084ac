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
// Kernel design (gfx950, wave64): one workgroup per 6 consecutive new rows of
// a sequence (12 waves, three per SIMD), a wave pair per row. The workgroup
// walks the rows' pages once:
//  * each page's record bytes (5,888) are loaded coalesced two pages ahead,
//    staged in LDS, and dequantized once for all six rows into an fp16 page
//    image (16 keys x 576 dims, rows placed so that both the row-slice reads
//    of QK^T and the transposed reads of PV are bank-conflict-free): the
//    latent as e2m1 * group scale (exact in fp16), the RoPE part as its e4m3
//    value; keys past the sequence end become zeros;
//  * the two waves of a pair split the dims as the decode does (256 latent +
//    32 RoPE each for QK^T, v_mfma_f32_16x16x32_f16 with A from the image and
//    B = fp16 Q*2^k in registers; 256 latent dims each for PV,
//    v_mfma_f32_16x16x16_f16 with A = V^T by ds_read_b64_tr_b16); the half
//    scores meet through LDS across the step's one barrier, and both waves
//    run the same softmax;
//  * the softmax is the decode's: an integer-valued lazy running max (slack
//    8, log2 units) and the largest outer-scale exponent Gs, so P =
//    2^(x - m) s2 2^-Gs <= 2^8 fits fp16 and rescales are powers of two;
//  * one barrier per page, between the half-score exchange and the softmax:
//    before it, the dequant of page k+1, the staging of page k+2 and QK^T of
//    page k; after it, softmax and PV of page k. Three image buffers keep
//    the dequant of page k+1 clear of PV readers of page k-2.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kRows = 6;                   // query rows per workgroup (4: 5.4-5.5 ms, 6: 5.0-5.2 ms)
constexpr int kWaves = 2 * kRows;
constexpr int kThreads = 64 * kWaves;
constexpr int kRec = 368;
constexpr int kLat = 512;
constexpr int kDqk = 576;
constexpr int kHeads = 16;
// Page image rows: key r's 576 fp16 at byte 1,184 r + 16 (r >> 3). The row
// stride is 296 dwords (an odd multiple of 8 banks) and keys 8..15 sit 4 banks
// further, so a QK^T row-slice read (16 keys x 4 dwords) and a transposed PV
// read (8 keys x 8 dwords per pass) each cover the 64 banks once.
constexpr int kImgRow = 2 * kDqk + 32;
constexpr int kImgBytes = 16 * kImgRow + 16;
__device__ __forceinline__ int img_row(int r) { return r * kImgRow + 16 * (r >> 3); }
constexpr int kPageBytes = 16 * kRec;
constexpr int kRawChunks = kPageBytes / 16;            // 368 16-byte chunks per page
constexpr int kImgChunks = 16 * (kDqk / 8);            // 1,152 fp16 chunks of 8 per page
constexpr float kTau = 8.0f;
constexpr int kGUnset = -(1 << 20);

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

struct __align__(16) PrefillMlaSmem {
  uint8_t img[3][kImgBytes];
  uint8_t raw[2][kPageBytes];
  v4f xch[2][kWaves][64];       // half scores: [step parity][wave][lane]
  float s2[3][16];
};

__device__ __forceinline__ uint32_t h2_bits(v2h x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }

__global__ __launch_bounds__(kThreads) void mla_prefill_kernel(DecodeMlaLaunch a) {
  __shared__ PrefillMlaSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave >> 1;            // this pair's row in the tile
  const int half = wave & 1;           // latent dims 256*half .. +256, RoPE 32*half .. +32
  const int row = lane & 15;
  const int grp = lane >> 4;

  const int tiles = (a.max_q_len + kRows - 1) / kRows;
  const int b = blockIdx.x / tiles;
  const int r0 = (blockIdx.x - b * tiles) * kRows;
  const int q0 = a.cu_q_lens[b];
  const int lq = a.cu_q_lens[b + 1] - q0;
  if (r0 >= lq) return;                                  // the whole workgroup
  const int L = a.seq_lens[b];
  const bool row_ok = r0 + rw < lq;
  const int pos = L - lq + r0 + rw;                      // this row's position (< 0: no key)
  const int pos_max = L - lq + min(lq, r0 + kRows) - 1;  // the tile's last row
  const int npages = pos_max >= 0 ? (pos_max >> 4) + 1 : 0;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;
  const size_t qrow = (size_t)q0 + r0 + rw;

  // ---- record bytes: thread t < 368 moves chunk t of a page
  auto load_page = [&](int p) -> v4u {
    v4u r = v4u{0u, 0u, 0u, 0u};
    if (p < npages && tid < kRawChunks)
      r = __builtin_nontemporal_load((const v4u *)(a.records + (size_t)bt[p] * kPageBytes + 16 * tid));
    return r;
  };
  auto stash_page = [&](const v4u &r, int buf) {
    if (tid < kRawChunks) *(v4u *)(sm.raw[buf] + 16 * tid) = r;
  };
  // ---- fp16 image of page p (staging buffer p & 1, image buffer p % 3;
  // keys past L: zeros)
  auto dequant = [&](int p) {
    const uint8_t *raw = sm.raw[p & 1];
    const int buf = p % 3;
    uint8_t *img = sm.img[buf];
#pragma unroll
    for (int c0 = 0; c0 < kImgChunks; c0 += kThreads) {
      const int c = c0 + tid;
      if (c >= kImgChunks) break;
      const int r = c / (kDqk / 8);
      const int j = c - r * (kDqk / 8);
      uint4 x = make_uint4(0, 0, 0, 0);
      if (p * 16 + r < L) {
        const uint8_t *rec = raw + r * kRec;
        if (j < kLat / 8) {
          const uint32_t w = *(const uint32_t *)(rec + 4 * j);
          const _Float16 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)rec[256 + (j >> 1)], 1.0f, false)[0];
          const v2h s2v = v2h{s, s};
          x = make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2v),
                         h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2v),
                         h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2v),
                         h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2v));
        } else {
          const uint2 w = *(const uint2 *)(rec + 304 + 8 * (j - kLat / 8));
          x = make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false)),
                         h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true)),
                         h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false)),
                         h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true)));
        }
      }
      *(uint4 *)(img + img_row(r) + 16 * j) = x;
    }
    if (tid < 16) sm.s2[buf][tid] = p * 16 + tid < L ? *(const float *)(raw + tid * kRec + 292) : 0.0f;
  };

  v4u nxt = load_page(0), nxt2 = load_page(1);

  // ---- Q of this row: the head's power of two k from all 576 dims (its
  // largest element times 2^k in [2^13, 2^14)); this lane keeps (head `row`,
  // grp) dims 256*half + 32c + 8*grp (c < 8) and 512 + 32*half + 8*grp (c = 8)
  // as fp16 Q * 2^k
  uint4 qop[9];
  int kexp = 0;
  {
    const uint4 *qp = (const uint4 *)(a.q + (qrow * a.hq + row) * kDqk + 8 * grp);
    uint4 qv[18];
#pragma unroll
    for (int c = 0; c < 18; ++c) qv[c] = row_ok ? qp[4 * c] : make_uint4(0, 0, 0, 0);
    uint32_t am = 0;
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      const uint32_t w[4] = {qv[c].x, qv[c].y, qv[c].z, qv[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
    am = max(am, (uint32_t)__shfl_xor((int)am, 16, 64));
    am = max(am, (uint32_t)__shfl_xor((int)am, 32, 64));
    kexp = am == 0 ? 0 : 14 - __builtin_amdgcn_frexp_expf(__uint_as_float(am << 16));
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const uint4 v = c < 8 ? (half ? qv[8 + c] : qv[c]) : (half ? qv[17] : qv[16]);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = h2_bits(v2h{(_Float16)__builtin_ldexpf(bf16lo(w[i]), kexp), (_Float16)__builtin_ldexpf(bf16hi(w[i]), kexp)});
      qop[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  const float c_score = __builtin_ldexpf(a.scale_log2, -kexp);
  const float c_rope = a.rope_scale * c_score;

  // prologue: page 0 dequantized, page 1 staged, pages 2 and 3 in flight
  stash_page(nxt, 0);
  __syncthreads();
  if (npages > 0) dequant(0);
  stash_page(nxt2, 1);
  nxt = load_page(2);
  nxt2 = load_page(3);
  __syncthreads();

  float m_run = -INFINITY;
  float l_run = 0.0f;
  int Gs = kGUnset;
  v4f o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // QK^T A operand: key `row`, latent dims 256*half + 32c + 8*grp, RoPE dims
  // 512 + 32*half + 8*grp; PV A operand (transposed): lane s of group grp
  // reads key 4*grp + s/4, dims 256*half + 16q + 4(s%4)
  const int a_off = img_row(row) + 512 * half + 16 * grp;
  const int r_off = img_row(row) + 2 * kLat + 64 * half + 16 * grp;
  const int t_off = img_row(4 * grp + (row >> 2)) + 2 * (256 * half + 4 * (row & 3));

  for (int k = 0; k < npages; ++k) {
    const int cur = k % 3;
    const bool active = row_ok && k * 16 <= pos;   // the same for both waves of a pair
    // ---- before the barrier: next page's image, staging, this page's QK^T
    if (k + 1 < npages) dequant(k + 1);
    stash_page(nxt, k & 1);           // page k+2 into the staging buffer page k has left
    nxt = nxt2;
    nxt2 = load_page(k + 4);
    const uint8_t *img = sm.img[cur];
    if (active) {
      v4f acc_l = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 x = *(const uint4 *)(img + a_off + 64 * c);
        acc_l = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x), __builtin_bit_cast(v8h, qop[c]),
                                                       acc_l, 0, 0, 0);
      }
      const uint4 xr = *(const uint4 *)(img + r_off);
      const v4f acc_r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xr),
                                                               __builtin_bit_cast(v8h, qop[8]),
                                                               v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      v4f y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = fmaf(c_score * sm.s2[cur][4 * grp + i], acc_l[i], c_rope * acc_r[i]);
      sm.xch[k & 1][wave][lane] = y;
    }
    __syncthreads();
    // ---- after the barrier: softmax and PV of this page
    if (active) {
      const float s2r = sm.s2[cur][row];
      const int e2 = __builtin_amdgcn_frexp_expf(s2r);
      if (__ballot(s2r > 0.0f && e2 > Gs)) {
        int emax = s2r > 0.0f ? e2 : kGUnset;
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) emax = max(emax, __shfl_xor(emax, msk, 64));
        const int g_new = __builtin_amdgcn_readfirstlane(emax);
        if (g_new != Gs) {
          const float f = __builtin_ldexpf(1.0f, max(Gs - g_new, -200));
#pragma unroll
          for (int q = 0; q < 16; ++q) o[q] *= f;
          Gs = g_new;
        }
      }
      const v4f y0 = sm.xch[k & 1][2 * rw][lane];
      const v4f y1 = sm.xch[k & 1][2 * rw + 1][lane];
      float x[4], s2p[4];
      bool raise_m = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * grp + i;
        x[i] = y0[i] + y1[i];
        if (k * 16 + key > pos) x[i] = -INFINITY;
        s2p[i] = __builtin_ldexpf(sm.s2[cur][key], -Gs);   // < 1
        raise_m |= x[i] > m_run + kTau;
      }
      if (__ballot(raise_m)) {
        float bmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        bmax = xor_max(xor_max(bmax, 16), 32);
        if (bmax > m_run + kTau) {
          const float m_new = __builtin_ceilf(bmax);
          const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int q = 0; q < 16; ++q) o[q] *= alpha;
          m_run = m_new;
        }
      }
      float pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pe = __builtin_amdgcn_exp2f(x[i] - m_run);   // <= 2^8
        l_run += pe;
        pw[i] = pe * s2p[i];
      }
      const v4h pb = v4h{(_Float16)pw[0], (_Float16)pw[1], (_Float16)pw[2], (_Float16)pw[3]};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const v4s va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s *)(img + t_off + 32 * q));
        o[q] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, va), pb, o[q], 0, 0, 0);
      }
    }
  }

  if (!row_ok) return;
  // out = 2^Gs O_acc / l (zeros when no key contributed)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  float sc = 0.0f;
  if (l_run > 0.0f && Gs != kGUnset) sc = __builtin_ldexpf(1.0f / l_run, Gs);
  uint16_t *dst = a.out + (qrow * a.hq + row) * kLat + 256 * half + 4 * grp;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    uint2 w;
    w.x = f32_to_bf16_bits(o[q][0] * sc) | (f32_to_bf16_bits(o[q][1] * sc) << 16);
    w.y = f32_to_bf16_bits(o[q][2] * sc) | (f32_to_bf16_bits(o[q][3] * sc) << 16);
    *(uint2 *)(dst + 16 * q) = w;
  }
}

}  // namespace

hipError_t launch_prefill_mla(const DecodeMlaLaunch &a, int max_seq_len, hipStream_t s) {
  (void)max_seq_len;
  if (a.hq != kHeads || a.cu_q_lens == nullptr || a.max_q_len <= 0) return hipErrorInvalidValue;
  const size_t tiles = (size_t)(a.max_q_len + kRows - 1) / kRows;
  hipLaunchKernelGGL(mla_prefill_kernel, dim3((unsigned)((size_t)a.batch * tiles)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
