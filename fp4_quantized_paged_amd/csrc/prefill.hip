// fp8 (e4m3) chunked-prefill attention over the paged cache.
//
// What is computed is the decode attention of vLLM PR 54705 ("Purpose",
// query-quantization and descale-handling bullets) for many new tokens at
// once: query i of a sequence with Lq new tokens and L keys sits at position
// L - Lq + i and attends keys j <= position (and > position - window); the
// QK descale is folded into the softmax scale and the exact bf16 relative bias
// bf16(slope_h * -(p - j)) is added after it; the V descale multiplies the
// output. The evidence document's "Tier 1" chunked-prefill case is the shape
// this serves.
//
// Kernel design (gfx950, wave64, 8 waves per workgroup):
//  * a workgroup owns 32 consecutive new tokens of one sequence and up to 8
//    query heads of one KV head (one wave per head); every wave holds two
//    16-token column blocks, so one staged K/V block feeds 16 QK^T MFMAs and
//    32 PV MFMAs per wave;
//  * K/V advance in 128-key blocks (8 pages). The workgroup copies a block's K
//    rows and token-minor V^T pages into LDS once (K rows bank-swizzled) while
//    the next block's bytes are already in flight in registers;
//  * QK^T and PV use v_mfma_f32_16x16x128_f8f6f4 with the same lane mapping as
//    decode: the key rows are permuted so that the S^T output lane of query row
//    (l % 16) holds exactly the 32 keys PV consumes from it, P = 2^8 p split
//    into two e4m3 terms;
//  * the bf16 bias of a block takes at most 159 distinct distances per head;
//    each wave fills a small LDS table of them and looks the scores' bias up;
//  * workgroups are numbered so that all tiles of one (sequence, KV head) land
//    on the same XCD (dispatch is round-robin over the 8 XCDs), where they
//    stream the same K/V blocks through that XCD's L2.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kPW = 8;            // waves per workgroup
constexpr int kTileTok = 32;      // new tokens per workgroup
constexpr int kBlkKeys = 128;     // keys per block (8 pages)
constexpr int kD = 128;           // head dim
constexpr int kKBytes = kBlkKeys * kD;          // 16 KB of K rows per block
constexpr int kVBytes = kBlkKeys * kD;          // 16 KB of V^T per block
constexpr int kBiasN = 160;                     // bias table entries per wave
constexpr int kLoadChunks = (kKBytes + kVBytes) / 16 / (64 * kPW);  // 16-byte chunks per thread

// Swizzle of the 16-byte column chunks of a K row in LDS: the 8 lanes that
// read one row chunk together (rows kidx = 32*(m/4) + const + m%4) hit 8
// different chunk slots, i.e. all 64 banks once.
__device__ __forceinline__ int kswz(int kidx) { return (kidx & 3) | (((kidx >> 5) & 1) << 2); }

struct PrefillSmem {
  uint8_t k[kKBytes];           // [128 keys][8 chunks of 16 B], chunk c at slot c ^ kswz(key)
  uint8_t v[kVBytes];           // [8 pages][128 dims][16 tokens]
  float bias[kPW][kBiasN];      // per wave: bias * log2(e) by distance
};

__global__ __launch_bounds__(64 * kPW) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_e4m3_kernel(PrefillE4M3Launch a, int tiles, int units, int head_blocks) {
  __shared__ PrefillSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane & 15;
  const int grp = lane >> 4;

  // ---- work item: XCD-major numbering (workgroup i runs on XCD i % 8)
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int u = xcd + 8 * (slot / tiles);
  const int tile = slot % tiles;
  if (u >= units) return;
  const int hb = u % head_blocks;
  const int g = (u / head_blocks) % a.hkv;
  const int b = u / (head_blocks * a.hkv);
  const int q0 = a.cu_q_lens[b];
  const int lq = a.cu_q_lens[b + 1] - q0;
  if (tile * kTileTok >= lq) return;
  const int L = a.seq_lens[b];
  const int ntok = min(kTileTok, lq - tile * kTileTok);
  const int P0 = L - lq + tile * kTileTok;        // position of the tile's first token
  const int group = a.hq / a.hkv;
  const int hloc = hb * kPW + wave;
  const bool head_ok = hloc < group;
  const int head = g * group + (head_ok ? hloc : 0);

  // keys [klo, khi): the union of the tile rows' ranges
  const int khi = P0 + ntok;
  const int klo = a.window > 0 ? max(0, P0 - a.window + 1) : 0;
  const int blk_lo = klo >> 7;
  const int blk_hi = (khi - 1) >> 7;              // inclusive
  const int page_last = (L - 1) >> 4;

  // ---- Q operands of this wave's two 16-token column blocks
  v8i qop[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    qop[cb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    const int r = cb * 16 + row;
    if (head_ok && r < ntok) {
      const uint4 *qp = (const uint4 *)(a.q + ((size_t)(q0 + tile * kTileTok + r) * a.hq + head) * kD + grp * 32);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint2 w = quant8_e4m3(qp[c], a.q_inv);
        qop[cb][2 * c] = (int)w.x;
        qop[cb][2 * c + 1] = (int)w.y;
      }
    }
  }
  const bool has_bias = a.slopes != nullptr;
  const float slope = has_bias ? a.slopes[head] : 0.0f;

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.0f, 0.0f};
  v4f o[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int t = 0; t < 8; ++t) o[cb][t] = v4f{0.f, 0.f, 0.f, 0.f};

  const size_t head_stride = (size_t)16 * kD;
  const size_t page_stride = (size_t)a.hkv * head_stride;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;

  // ---- block loader: thread chunk q in [0, 2048): q < 1024 -> K, else V^T;
  // 128 chunks (2 KB) per page. Pages past the sequence end are clamped.
  uint4 pre[kLoadChunks];
  auto load_block = [&](int blk) {
#pragma unroll
    for (int c = 0; c < kLoadChunks; ++c) {
      const int q = tid + c * 64 * kPW;
      const int tensor = q >> 10;
      const int pg = (q >> 7) & 7;
      const int off = (q & 127) << 4;
      const int page = min(blk * 8 + pg, page_last);
      const uint8_t *base = tensor == 0 ? a.kc : a.vc;
      const v4u x = __builtin_nontemporal_load(
          (const v4u *)(base + (size_t)bt[page] * page_stride + (size_t)g * head_stride + off));
      pre[c] = make_uint4(x.x, x.y, x.z, x.w);
    }
  };
  auto stash_block = [&](int blk) {
    // positions outside [klo, L) get zero V bytes (stale or poisoned pages,
    // and 0 * NaN would poison the MFMA)
    const int j0 = blk * kBlkKeys;
    const bool edge = j0 < klo || j0 + kBlkKeys > L;
#pragma unroll
    for (int c = 0; c < kLoadChunks; ++c) {
      const int q = tid + c * 64 * kPW;
      const int tensor = q >> 10;
      const int pg = (q >> 7) & 7;
      const int off = (q & 127) << 4;
      if (tensor == 0) {
        const int kidx = pg * 16 + (off >> 7);       // key row within the block
        const int chunk = (off >> 4) & 7;
        *(uint4 *)(sm.k + kidx * kD + ((chunk ^ kswz(kidx)) << 4)) = pre[c];
      } else {
        uint4 x = pre[c];
        if (edge) {
          const int pos0 = j0 + pg * 16;            // 16 tokens of one dim
          uint32_t mk[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t mv = 0;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
              const int p = pos0 + 4 * w + bb;
              mv |= (p >= klo && p < L) ? (0xFFu << (8 * bb)) : 0u;
            }
            mk[w] = mv;
          }
          x.x &= mk[0]; x.y &= mk[1]; x.z &= mk[2]; x.w &= mk[3];
        }
        *(uint4 *)(sm.v + pg * 2048 + off) = x;
      }
    }
  };

  const float fold = a.fold_log2;
  if (blk_lo <= blk_hi) load_block(blk_lo);   // empty when seq_lens < new tokens
  for (int blk = blk_lo; blk <= blk_hi; ++blk) {
    __syncthreads();                  // everyone is done reading the previous block
    stash_block(blk);
    __syncthreads();
    if (blk < blk_hi) load_block(blk + 1);
    const int j0 = blk * kBlkKeys;

    // ---- per-wave bias table for this block: entry e <-> distance
    // d = (P0 - j0) + e - 127, value bf16(slope * -d) * log2(e)
    if (has_bias) {
      for (int e = lane; e < kBiasN; e += 64) {
        const float d = (float)(P0 - j0 + e - 127);
        sm.bias[wave][e] = round_bf16_finite(slope * -d) * kLog2e;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    const bool edge = (j0 + kBlkKeys - 1 > P0) || (a.window > 0 && j0 < khi - a.window);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      v8i phi, plo;
      // ---- S^T = K Q^T: lane (row, grp) gets keys
      // kidx = 32*grp + 16*(j/4) + 4*(j%4) + i of query row (cb*16 + row)
      v4f s[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kidx = 32 * (row >> 2) + 16 * (j >> 2) + 4 * (j & 3) + (row & 3);
        const int c0 = 2 * grp;
        const uint4 x0 = *(const uint4 *)(sm.k + kidx * kD + (((c0) ^ kswz(kidx)) << 4));
        const uint4 x1 = *(const uint4 *)(sm.k + kidx * kD + (((c0 + 1) ^ kswz(kidx)) << 4));
        const v8i kop = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        s[j] = mfma_16x16x128_e4m3(kop, qop[cb], v4f{0.f, 0.f, 0.f, 0.f});
      }
      const int r = cb * 16 + row;
      // This lane's keys are j0 + 32*grp + c, c = 16*(j/4) + 4*(j%4) + i in
      // [0, 32). Bias entry r - kidx + 127 = tb_base + (31 - c) with
      // tb_base >= 0, so every lookup is an immediate LDS offset.
      const float *tb = &sm.bias[wave][r - 32 * grp + 96];
      const int c_hi = P0 + r - j0 - 32 * grp;              // keys with c <= c_hi are causal
      const int c_lo = a.window > 0 ? c_hi - a.window : -1;  // and c > c_lo inside the window
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * (j >> 2) + 4 * (j & 3) + i;
          float x = has_bias ? fmaf(s[j][i], fold, tb[31 - c]) : s[j][i];
          if (edge) x = (c <= c_hi && c > c_lo) ? x : -INFINITY;
          s[j][i] = x;
        }
      float bmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[j][i]);
      bmax = wave_max_xor(bmax, 16);
      bmax = wave_max_xor(bmax, 32);
      const float scale = has_bias ? 1.0f : fold;
      const float m_new = fmaxf(m_run[cb], bmax * scale);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_use);
      m_run[cb] = m_new;
      const float off = 8.0f - m_use;
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(fmaf(s[j][i], scale, off));
          psum += pv[i];
        }
        const uint32_t hi = cvt4_e4m3(pv[0], pv[1], pv[2], pv[3]);
        const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
        const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
        phi[j] = (int)hi;
        plo[j] = (int)cvt4_e4m3(pv[0] - h01.x, pv[1] - h01.y, pv[2] - h23.x, pv[3] - h23.y);
      }
      l_run[cb] = l_run[cb] * alpha + psum;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) o[cb][t] *= alpha;
      }
      // ---- O^T += V^T P^T: tile t covers dims 16t .. 16t+15
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int dim = 16 * t + row;
        const uint4 x0 = *(const uint4 *)(sm.v + (2 * grp) * 2048 + dim * 16);
        const uint4 x1 = *(const uint4 *)(sm.v + (2 * grp + 1) * 2048 + dim * 16);
        const v8i vop = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        o[cb][t] = mfma_16x16x128_e4m3(vop, phi, o[cb][t]);
        o[cb][t] = mfma_16x16x128_e4m3(vop, plo, o[cb][t]);
      }
      // keep the two column blocks' work apart: interleaving them doubles
      // the live scores and operands
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- normalise and write bf16 rows: lane holds O[row][16t + 4*grp + i]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    float l = l_run[cb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = cb * 16 + row;
    if (!head_ok || r >= ntok) continue;
    const float f = l > 0.0f ? a.v_scale / l : 0.0f;
    uint16_t *dst = a.out + ((size_t)(q0 + tile * kTileTok + r) * a.hq + head) * kD + 4 * grp;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t lo = f32_to_bf16_bits(o[cb][t][0] * f) | (f32_to_bf16_bits(o[cb][t][1] * f) << 16);
      const uint32_t hi = f32_to_bf16_bits(o[cb][t][2] * f) | (f32_to_bf16_bits(o[cb][t][3] * f) << 16);
      *(uint2 *)(dst + 16 * t) = make_uint2(lo, hi);
    }
  }
}

}  // namespace

hipError_t launch_prefill_e4m3(const PrefillE4M3Launch &a, hipStream_t s) {
  if (a.d != kD) return hipErrorNotSupported;
  const int group = a.hq / a.hkv;
  const int head_blocks = (group + kPW - 1) / kPW;
  const int units = a.batch * a.hkv * head_blocks;
  const int tiles = (a.max_q_len + kTileTok - 1) / kTileTok;
  if (tiles == 0) return hipSuccess;
  const size_t grid = (size_t)8 * ((units + 7) / 8) * tiles;
  hipLaunchKernelGGL(prefill_e4m3_kernel, dim3((unsigned)grid), dim3(64 * kPW), 0, s, a, tiles, units,
                     head_blocks);
  return hipGetLastError();
}

}  // namespace kvq
