// fp8 (e4m3) paged decode attention: split-KV kernel and split combine.
//
// What is computed (vLLM PR 54705, "Purpose", query-quantization and
// descale-handling bullets): Q is quantized to e4m3 with its per-tensor scale;
// raw scores are e4m3 dot products; the QK descale is folded into the softmax
// scale and the exact bf16 relative bias is added after it (bf16(slope_h *
// -(p - j)), or the entry T[h][min(p - j, E - 1)] of a learned table: the
// page's "Environment" and "Test Plan" sections, extents 128 and 1024; blocks
// entirely beyond the extent add the last entry without lookups); the V
// descale multiplies the output. Online softmax across key blocks follows the
// evidence document's "Tier 0" (P in fp8, pre-scaled by 2^8 so its largest
// value 256 stays below the e4m3 maximum; rescaling is exact here, i.e. a
// threshold of 0).
//
// Kernel design (gfx950, wave64):
//  * one workgroup per (sequence, KV head, 16-row query tile, split), with W
//    waves that take interleaved 128-key blocks (8 pages) of the split;
//  * QK^T: per block, eight v_mfma_f32_16x16x128_f8f6f4 with A = 16 key rows
//    (K = head_dim) and B = the 16 query rows of the GQA group. The key row
//    each lane loads is permuted so that the output lane holding query row
//    (l % 16) receives exactly the 32 keys of pages {2g, 2g+1} of the block,
//    g = l / 16: that is the B-operand slice PV needs, so P never leaves the
//    registers;
//  * PV: A = V^T, read straight from the token-minor V pages (16 contiguous
//    bytes per dim per page), B = P. P = 256 * p is split into two e4m3 terms
//    (hi = e4m3(P), lo = e4m3(P - hi)) accumulated by two MFMAs, which keeps
//    the relative error of each weight near 2^-8 while staying on fp8 MFMA;
//    a ones tile in the same MFMA stream sums the two terms into the
//    normaliser, so a weight too small for both terms is dropped from the
//    numerator and the denominator alike;
//  * V^T operands come straight from HBM with 16-byte loads (the cache
//    layout makes each operand slice contiguous). With head_dim 128 the K
//    rows of a block are fetched as whole 128-byte lines into a per-wave LDS
//    area and read back in the permuted operand order; head_dim 64 loads its
//    K operand slices directly;
//  * the page ids of a block are fetched one block ahead, one vector load for
//    all eight pages, so that the K and V loads of a block are issued back to
//    back with no block-table round trip in front of them;
//  * W waves merge through LDS with a single barrier; with one split the
//    workgroup writes bf16 out directly, otherwise (m, l, o) partials go to
//    the workspace and the combine kernel merges them.
#include "kvq_combine.h"
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

template <int D>
struct DecodeTile {
  static constexpr int kTiles = D / 16;   // 16-dim output tiles
};

// Byte mask (0xFF per kept byte) of the 16 tokens of a page: tokens whose
// absolute position lies in [lo, hi) are kept.
__device__ __forceinline__ void page_byte_mask(int page_pos0, int lo, int hi, uint32_t m[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int p = page_pos0 + 4 * w + b;
      v |= (p >= lo && p < hi) ? (0xFFu << (8 * b)) : 0u;
    }
    m[w] = v;
  }
}

// LDS of one workgroup: one area per wave, its K staging (head_dim 128,
// 16 KB) during the key loop and its unnormalised O ([16][D + 4] fp32; the
// 16-byte row pad spreads each 8-lane group of 16-byte writes over all
// banks) at the merge; then [W][16] m and l.
template <int D, int W>
struct DecodeSmem {
  static constexpr int kStageBytes = D == 128 ? 16384 : 0;
  static constexpr int kOStride = D + 4;
  static constexpr int kOBytes = 16 * kOStride * 4;
  static constexpr int kWaveBytes = kStageBytes > kOBytes ? kStageBytes : kOBytes;
  static constexpr int kRegion = W * kWaveBytes;
  static constexpr int kBytes = kRegion + 2 * W * 16 * 4;
};

template <int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void decode_e4m3_kernel(DecodeE4M3Launch a, int splits,
                                                            int blocks_per_split, int qtiles) {
  constexpr int kTiles = DecodeTile<D>::kTiles;
  using Sm = DecodeSmem<D, W>;
  __shared__ __align__(16) uint8_t smem[Sm::kBytes];
  float *s_m = (float *)(smem + Sm::kRegion);
  float *s_l = s_m + W * 16;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;      // query row (B/N index) and A-row index
  const int grp = lane >> 4;      // K-slice / key-group index

  int idx = blockIdx.x;
  const int split = idx % splits;
  idx /= splits;
  const int qt = idx % qtiles;
  idx /= qtiles;
  const int g = idx % a.hkv;
  const int b = idx / a.hkv;

  const int group = a.hq / a.hkv;
  const int qrow = qt * 16 + row;
  const bool qvalid = qrow < group;
  const int head = g * group + (qvalid ? qrow : 0);

  const int L = a.seq_lens[b];
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int page_lo = lo >> 4;
  const int page_hi = (L + 15) >> 4;
  const int nblk = (page_hi - page_lo + 7) >> 3;
  const int blk_begin = split * blocks_per_split;
  const int blk_end = min(nblk, blk_begin + blocks_per_split);

  // ---- Q: quantize this lane's 32 dims of its query row to e4m3
  v8i qop = {0, 0, 0, 0, 0, 0, 0, 0};
  if (qvalid && (D == 128 || grp < 2)) {
    const uint4 *qp = (const uint4 *)(a.q + ((size_t)b * a.hq + head) * D + grp * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint2 w = quant8_e4m3(qp[c], a.q_inv);
      qop[2 * c] = (int)w.x;
      qop[2 * c + 1] = (int)w.y;
    }
  }
  const float slope = (a.slopes != nullptr && qvalid) ? a.slopes[head] : 0.0f;
  // learned table: this head's row; distances from rel_extent - 1 on read
  // its last entry (kept pre-multiplied by log2(e) for the far blocks)
  const uint16_t *rel_row = a.rel != nullptr ? a.rel + (size_t)head * a.rel_extent : nullptr;
  const float rel_last = rel_row != nullptr ? __uint_as_float((uint32_t)rel_row[a.rel_extent - 1] << 16) * kLog2e : 0.0f;
  const bool has_bias = a.slopes != nullptr || a.rel != nullptr;
  const float qpos = (float)(L - 1);

  float m_run = -INFINITY;   // running max, log2 domain
  // row sums of P as PV sums them (a ones tile on fp8 MFMA over both e4m3
  // terms): every element of lane (row, grp) holds the sum for query `row`
  v4f ol = v4f{0.f, 0.f, 0.f, 0.f};
  const v8i ones8 = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0
  v4f o[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};

  const size_t kv_head_stride = (size_t)16 * D;               // bytes per head-page
  const size_t page_stride = (size_t)a.hkv * kv_head_stride;  // bytes per page
  const size_t g_off = (size_t)g * kv_head_stride;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;

  // Fused append: the current token (position L - 1, in the last block) is
  // quantized with the store's quantizer and written into its page by the
  // wave that reads that block. Its bf16 K/V and page id are requested here;
  // the bytes are written once the wave's first block has its loads in
  // flight (so the wave starts as early as the others), or before those
  // loads when that first block is the last one. With several query tiles
  // each tile's workgroup writes the same bytes.
  const int blk_last = nblk - 1;
  const int blk_first = blk_begin + wave;   // this wave's first block
  const bool appender = a.k_new != nullptr && L > 0 && blk_last >= blk_begin && blk_last < blk_end &&
                        wave == (blk_last - blk_begin) % W;
  const bool app_lane = appender && lane < D / 8;
  uint4 k_tok = make_uint4(0u, 0u, 0u, 0u), v_tok = k_tok;
  int app_page = 0;
  if (app_lane) {
    const size_t src = ((size_t)b * a.hkv + g) * D + 8 * lane;
    k_tok = *(const uint4 *)(a.k_new + src);
    v_tok = *(const uint4 *)(a.v_new + src);
    app_page = bt[(L - 1) >> 4];
  }
  auto append = [&]() {
    if (app_lane) {
      const int pos = L - 1;
      const size_t base = (size_t)app_page * page_stride + g_off;
      const uint2 kq = quant8_e4m3(k_tok, a.k_inv);
      const uint2 vq = quant8_e4m3(v_tok, a.v_inv);
      *(uint2 *)(a.kc_w + base + (size_t)(pos & 15) * D + 8 * lane) = kq;
      uint8_t *vdst = a.vc_w + base + (pos & 15) + 16 * (8 * lane);   // token-minor: dim d at 16 d
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vdst[16 * i] = (uint8_t)(vq.x >> (8 * i));
        vdst[16 * (4 + i)] = (uint8_t)(vq.y >> (8 * i));
      }
    }
  };

  // head_dim 128: lane l holds the physical page of page (l & 7) of the next
  // block, clamped to the sequence's last page.
  int pid_next = 0;
  if constexpr (D == 128) {
    if (blk_begin + wave < blk_end)
      pid_next = bt[min(page_lo + (blk_begin + wave) * 8 + (lane & 7), page_hi - 1)];
  }

  for (int blk = blk_begin + wave; blk < blk_end; blk += W) {
    if (appender && blk == blk_last) {
      if (blk == blk_first) append();
      // the appended bytes are in memory before this block's loads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    const int pbase = page_lo + blk * 8;
    // Pages this lane touches: K rows come from pages pbase + 2*(row/4) + {0,1},
    // V columns (and this lane's output keys) from pages pbase + 2*grp + {0,1}.
    // Pages past the sequence end are clamped to its last page: their keys are
    // masked and their V bytes zeroed below, so every load stays unconditional.
    const int vp0 = pbase + 2 * grp;
    const bool edge = (pbase * 16 < lo) || ((pbase + 8) * 16 > L);

    // ---- K operands: MFMA j takes token 4*(j%4) + (row%4) of page
    // pbase + 2*(row/4) + (j/4); V^T operands: tile t, dim 16t + row, 16
    // tokens of vp0 then of vp0+1
    v8i kop[8];
    v8i vop[kTiles];
    if constexpr (D == 128) {
      // Whole-line K loads through LDS: load i brings rows 8*(i&1) .. +8 of
      // block page i/2 (1 KB contiguous), 16-byte chunks XOR-swizzled by
      // (token & 3) and bit 1 of the page so that these row writes and the
      // operand reads below both hit 32 distinct banks per 8 lanes.
      const int pid = pid_next;
      int ph[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ph[i] = __builtin_amdgcn_readlane(pid, i);
      uint8_t *kst = smem + wave * Sm::kWaveBytes;
      v4u kl[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        kl[i] = __builtin_nontemporal_load(
            (const v4u *)(a.kc + (size_t)ph[i / 2] * page_stride + g_off + (8 * (i & 1) + (lane >> 3)) * 128 + 16 * (lane & 7)));
      const int vphys0 = grp == 0 ? ph[0] : grp == 1 ? ph[2] : grp == 2 ? ph[4] : ph[6];
      const int vphys1 = grp == 0 ? ph[1] : grp == 1 ? ph[3] : grp == 2 ? ph[5] : ph[7];
      const uint8_t *vb0 = a.vc + (size_t)vphys0 * page_stride + g_off + row * 16;
      const uint8_t *vb1 = a.vc + (size_t)vphys1 * page_stride + g_off + row * 16;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const v4u x0 = __builtin_nontemporal_load((const v4u *)(vb0 + 256 * t));
        const v4u x1 = __builtin_nontemporal_load((const v4u *)(vb1 + 256 * t));
        vop[t] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
      // next block's page ids (the last block re-reads its own)
      const int nblk_next = blk + W < blk_end ? blk + W : blk;
      pid_next = bt[min(page_lo + nblk_next * 8 + (lane & 7), page_hi - 1)];
      // keep all of the block's loads ahead of the LDS writes that wait on them
      __builtin_amdgcn_sched_barrier(0);
      if (blk == blk_first && blk != blk_last) append();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = (lane & 7) ^ ((lane >> 3) & 3) ^ (4 * ((i >> 2) & 1));
        *(v4u *)(kst + (i / 2) * 2048 + (8 * (i & 1) + (lane >> 3)) * 128 + 16 * slot) = kl[i];
      }
      const int rswz = (row & 3) | (((row >> 2) & 1) << 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint8_t *src = kst + (2 * (row >> 2) + (j >> 2)) * 2048 + (4 * (j & 3) + (row & 3)) * 128;
        const v4u x0 = *(const v4u *)(src + 16 * ((2 * grp) ^ rswz));
        const v4u x1 = *(const v4u *)(src + 16 * ((2 * grp + 1) ^ rswz));
        kop[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
    } else {
      const int kphys0 = bt[min(pbase + 2 * (row >> 2), page_hi - 1)];
      const int kphys1 = bt[min(pbase + 2 * (row >> 2) + 1, page_hi - 1)];
      const int vphys0 = bt[min(vp0, page_hi - 1)];
      const int vphys1 = bt[min(vp0 + 1, page_hi - 1)];
      const uint8_t *kb0 = a.kc + (size_t)kphys0 * page_stride + g_off + (row & 3) * D + grp * 32;
      const uint8_t *kb1 = a.kc + (size_t)kphys1 * page_stride + g_off + (row & 3) * D + grp * 32;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (grp < 2) {
          const uint8_t *src = (j < 4 ? kb0 : kb1) + 4 * (j & 3) * D;
          const v4u x0 = __builtin_nontemporal_load((const v4u *)src);
          const v4u x1 = __builtin_nontemporal_load((const v4u *)(src + 16));
          kop[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        } else {
          kop[j] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
      const uint8_t *vb0 = a.vc + (size_t)vphys0 * page_stride + g_off + row * 16;
      const uint8_t *vb1 = a.vc + (size_t)vphys1 * page_stride + g_off + row * 16;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const v4u x0 = __builtin_nontemporal_load((const v4u *)(vb0 + 256 * t));
        const v4u x1 = __builtin_nontemporal_load((const v4u *)(vb1 + 256 * t));
        vop[t] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
      if (blk == blk_first && blk != blk_last) append();
    }

    // ---- S^T = K Q^T: lane holds keys (vp0 + j/4, token 4*(j%4) + i) of its query row
    v4f sacc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sacc[j] = mfma_16x16x128_e4m3(kop[j], qop, v4f{0.f, 0.f, 0.f, 0.f});

    // ---- scores in the log2 domain: x = raw * fold (+ bias); masked keys -inf
    const int kpos0 = vp0 * 16;   // absolute position of this lane's first key
    if (rel_row != nullptr) {
      // keys of this block sit at distances L - 1 - kpos; a block whose
      // nearest key is at least rel_extent - 1 away reads only the last entry
      if ((L - 1) - (pbase * 16 + 127) >= a.rel_extent - 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[j][i] = fmaf(sacc[j][i], a.fold_log2, rel_last);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kpos = kpos0 + 16 * (j >> 2) + 4 * (j & 3) + i;
            const int e = min(max((L - 1) - kpos, 0), a.rel_extent - 1);   // later keys are masked
            const float bias = __uint_as_float((uint32_t)rel_row[e] << 16);
            sacc[j][i] = fmaf(sacc[j][i], a.fold_log2, bias * kLog2e);
          }
      }
    } else if (has_bias) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kpos = kpos0 + 16 * (j >> 2) + 4 * (j & 3) + i;
          const float bias = round_bf16_finite(slope * ((float)kpos - qpos));
          sacc[j][i] = fmaf(sacc[j][i], a.fold_log2, bias * kLog2e);
        }
    }
    if (edge) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kpos = kpos0 + 16 * (j >> 2) + 4 * (j & 3) + i;
          sacc[j][i] = (kpos >= lo && kpos < L) ? sacc[j][i] : -INFINITY;
        }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, sacc[j][i]);
    bmax = wave_max_xor(bmax, 16);
    bmax = wave_max_xor(bmax, 32);
    // without bias the max was taken on raw scores (fold > 0 keeps the order)
    const float scale = has_bias ? 1.0f : a.fold_log2;
    const float m_new = fmaxf(m_run, bmax * scale);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    // P = 2^8 p (exponent offset 8), split into two e4m3 terms
    const float off = 8.0f - m_use;
    v8i phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sacc[j][i], scale, off));
      const uint32_t hi = cvt4_e4m3(p[0], p[1], p[2], p[3]);
      const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
      const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
      phi[j] = (int)hi;
      plo[j] = (int)cvt4_e4m3(p[0] - h01.x, p[1] - h01.y, p[2] - h23.x, p[3] - h23.y);
    }

    // ---- zero V bytes of tokens outside [lo, L) (stale, NaN or clamped pages:
    // 0 * NaN would poison the MFMA)
    if (edge) {
      uint32_t m0[4], m1[4];
      page_byte_mask(vp0 * 16, lo, L, m0);
      page_byte_mask(vp0 * 16 + 16, lo, L, m1);
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vop[t][w] &= (int)m0[w];
          vop[t][w + 4] &= (int)m1[w];
        }
      }
    }

    // ---- O^T = V^T P^T, rescaled first when any row's max moved
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < kTiles; ++t) o[t] *= alpha;
      ol *= alpha;
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      o[t] = mfma_16x16x128_e4m3(vop[t], phi, o[t]);
      o[t] = mfma_16x16x128_e4m3(vop[t], plo, o[t]);
    }
    // the normaliser sums the same rounded terms as PV
    ol = mfma_16x16x128_e4m3(ones8, phi, ol);
    ol = mfma_16x16x128_e4m3(ones8, plo, ol);
  }
  const float l_run = ol[0];

  // ---- merge the W waves through LDS, in wave order (deterministic). Each
  // wave parks m, l and its unnormalised O (lane: query row, dims
  // 16t + 4*grp + i) in its own area, which no other wave touches during the
  // key loop, so one barrier suffices; then each thread finishes four dims of
  // one query row.
  {
    float *s_ow = (float *)(smem + wave * Sm::kWaveBytes);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) *(v4f *)(s_ow + row * Sm::kOStride + 16 * t + 4 * grp) = o[t];
  }
  if (grp == 0) {
    s_m[wave * 16 + row] = m_run;
    s_l[wave * 16 + row] = l_run;
  }
  __syncthreads();

  constexpr int kQuads = D / 4;
  const int rows_here = min(16, group - qt * 16);
  const bool out_vec = ((uintptr_t)a.out & 7) == 0;
  for (int e = threadIdx.x; e < rows_here * kQuads; e += 64 * W) {
    const int r = e / kQuads;
    const int dcol = 4 * (e - r * kQuads);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w * 16 + r]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w * 16 + r] - Mu);
      den += f * s_l[w * 16 + r];
      acc += f * *(const v4f *)((const float *)(smem + w * Sm::kWaveBytes) + r * Sm::kOStride + dcol);
    }
    const int h = g * group + qt * 16 + r;
    if (splits == 1) {
      uint16_t *dst = a.out + ((size_t)b * a.hq + h) * D + dcol;
      const uint32_t w0 = f32_to_bf16_bits(den > 0.0f ? (acc[0] / den) * a.v_scale : 0.0f) |
                          (f32_to_bf16_bits(den > 0.0f ? (acc[1] / den) * a.v_scale : 0.0f) << 16);
      const uint32_t w1 = f32_to_bf16_bits(den > 0.0f ? (acc[2] / den) * a.v_scale : 0.0f) |
                          (f32_to_bf16_bits(den > 0.0f ? (acc[3] / den) * a.v_scale : 0.0f) << 16);
      if (out_vec) {
        *(uint2 *)dst = uint2{w0, w1};
      } else {
        dst[0] = (uint16_t)w0;
        dst[1] = (uint16_t)(w0 >> 16);
        dst[2] = (uint16_t)w1;
        dst[3] = (uint16_t)(w1 >> 16);
      }
    } else {
      const size_t pi = ((size_t)b * a.hq + h) * splits + split;
      *(v4f *)(a.part_o + pi * D + dcol) = acc;
      if (dcol == 0) {
        a.part_ml[2 * pi] = M;
        a.part_ml[2 * pi + 1] = den;
      }
    }
  }
}

template <int D, int W>
hipError_t launch_decode_t(const DecodeE4M3Launch &a, const DecodePlan &p, hipStream_t s) {
  const size_t grid = (size_t)a.batch * a.hkv * p.qtiles * p.splits;
  hipLaunchKernelGGL((decode_e4m3_kernel<D, W>), dim3((unsigned)grid), dim3(64 * W), 0, s, a,
                     p.splits, p.blocks_per_split, p.qtiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL((split_combine_kernel<D>), dim3((unsigned)((size_t)a.batch * a.hq)), dim3(D * combine_groups(p.splits)), 0, s,
                     a.part_o, a.part_ml, a.out, p.splits, a.v_scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeE4M3Launch &a, const DecodePlan &p, hipStream_t s) {
  switch (p.waves) {
    case 1: return launch_decode_t<D, 1>(a, p, s);
    case 2: return launch_decode_t<D, 2>(a, p, s);
    case 4: return launch_decode_t<D, 4>(a, p, s);
    default: return launch_decode_t<D, 8>(a, p, s);
  }
}

}  // namespace

hipError_t launch_decode_e4m3(const DecodeE4M3Launch &a, const DecodePlan &p, hipStream_t s) {
  if (a.d == 64) return launch_decode_d<64>(a, p, s);
  return launch_decode_d<128>(a, p, s);
}

}  // namespace kvq
