// fp8 (e4m3) chunked-prefill attention over the paged cache.
//
// What is computed is the decode attention of vLLM PR 54705 ("Purpose",
// query-quantization and descale-handling bullets) for many new tokens at
// once: query i of a sequence with Lq new tokens and L keys sits at position
// L - Lq + i and attends keys j <= position (and > position - window); the
// QK descale is folded into the softmax scale and the exact bf16 relative bias
// is added after it: bf16(slope_h * -(p - j)), or the entry
// T[h][min(p - j, E - 1)] of a learned table (the page's "Environment" and
// "Test Plan": a learned relative position bias, extents 128 and 1024); the V
// descale multiplies the output. The evidence document's "Tier 1"
// chunked-prefill case is the shape this serves.
//
// Kernel design (gfx950, wave64, 8 waves per workgroup):
//  * a workgroup owns 32 consecutive new tokens of one sequence and up to 8
//    query heads of one KV head (one wave per head); under the slope bias it
//    owns one query head and up to 8 consecutive 32-token tiles instead (one
//    wave per tile), so that its waves stop at about the same block. Every
//    wave holds two 16-token column blocks, so one staged K/V block feeds 16
//    QK^T MFMAs and 32 PV MFMAs per wave;
//  * K/V advance in 128-key blocks (8 pages). The workgroup copies a block's K
//    rows (bank-swizzled) and its token-minor V^T pages, converted once to
//    fp16, into LDS while the next block's bytes are already in flight in
//    registers;
//  * QK^T uses v_mfma_f32_16x16x128_f8f6f4 with the same lane mapping as
//    decode: the key rows are permuted so that the S^T output lane of query row
//    (l % 16) holds exactly the 32 keys PV consumes from it;
//  * PV runs on v_mfma_f32_16x16x32_f16 with P in fp16 (exact e4m3 V, 11-bit
//    P mantissa, fp32 accumulation); a ones tile in the same MFMA stream
//    accumulates the row sums of the rounded P, so the normaliser matches
//    what PV summed;
//  * the bf16 bias of a block takes at most 159 distinct distances per head;
//    each wave fills a small LDS table of them (from the slope or from the
//    learned table) and looks the scores' bias up; with the learned table, a
//    block entirely beyond its extent adds the last entry instead;
//  * blocks run from the diagonal outward (nearest keys first), so a row
//    under a distance-decaying bias meets its largest scores first; the
//    running max is lazy (raised only when a score passes it by more than 8,
//    log2 units; fp16 P <= 2^8 keeps its relative precision), so O is rarely
//    rescaled; and a wave whose every P in a block would be exactly zero
//    (every exponent argument at least 26 below the running max: fp16 rounds
//    2^-26 to 0; with e4m3 P = 2^(x - m + 8), 19 below: e4m3 rounds 2^-11 to
//    0) skips that block's exp2 and PV, which leaves the result bit for bit
//    unchanged;
//    with the slope bias (non-negative slopes) a wave stops altogether once
//    a bound on every remaining score lies that far below the running max:
//    |q . k| <= 448 * sum |q| (448 is the e4m3 maximum), or, given the
//    per-block key norms that key_norm_kernel writes first, |q| times the
//    largest remaining key norm (Cauchy-Schwarz), and the bias only falls
//    with distance; the workgroup leaves the key loop when all of its waves
//    have stopped;
//  * the tile groups of each unit are spread over the 8 XCDs in chunks (the
//    same mix of units on every XCD), and units are ordered costliest first
//    with the sequences innermost, so that consecutive workgroups of an XCD,
//    which go to its shader engines in turn, cost about the same.
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
constexpr int kBiasN = 160;                     // bias table entries (distances) of a block
constexpr int kMaxPM = 1024;                    // slope bias: key-norm prefix maxima held in LDS
constexpr int kBiasWave = 736;                  // four copies per wave, one per lane group

// Lane group g reads its own copy of the wave's bias table, starting at entry
// bias_copy(g). One lookup has the 16 lanes of group g read 16 consecutive
// entries 32 g below group 0's; the copy bases (0, 208, 400, 576) put the
// four windows on disjoint banks whether the banks number 32 (two lane groups
// served together) or 64 (all four), where one shared copy conflicts 2-way.
__device__ __forceinline__ int bias_copy(int g) { return 192 * g + ((g == 1 || g == 2) ? 16 : 0); }
constexpr int kLoadChunks = (kKBytes + kVBytes) / 16 / (64 * kPW);  // 16-byte chunks per thread

// Swizzle of the 16-byte column chunks of a K row in LDS. The 16 lanes of one
// lane group read chunk c of rows kidx = 32*(m/4) + const + m%4, m = 0..15;
// with slot = c ^ kswz(kidx) they cover 16 distinct 16-byte bank groups of a
// 256-byte span (64 banks) and any 8 consecutive lanes 8 distinct groups of a
// 128-byte span, so a ds_read_b128 pass never repeats a bank.
__device__ __forceinline__ int kswz(int kidx) {
  return ((kidx & 3) | (((kidx >> 5) & 1) << 2)) ^ ((kidx >> 6) & 1);
}

struct __align__(16) PrefillSmem {
  uint4 k[kKBytes / 16];        // [128 keys][8 chunks of 16 B], chunk c at slot c ^ kswz(key)
  uint4 v[2 * kVBytes / 16];    // fp16 V^T: [8 pages][2 halves][128 dims][8 tokens];
                                // fp8-P variant: e4m3 V^T [8 pages][128 dims][16 tokens]
                                // in the first half
  float bias[kPW][kBiasWave];   // per wave: bias * log2(e) by distance, four copies
  __attribute__((aligned(16))) int done[2][kPW];   // slope bias: waves whose remaining blocks are all zero P
  float qbound[kPW][32];        // slope bias: per wave and query row, 448 * sum |q|
  float qnorm[kPW][32];         // slope bias: per wave and query row, |q| (Euclidean, codes)
  float pm[kMaxPM];             // slope bias: largest key norm of blocks blk_lo .. blk_lo + i
  float pmw[kPW];               // per-wave maxima of the prefix scan
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8h as_v8h(uint4 x) { return __builtin_bit_cast(v8h, x); }

// Two e4m3 bytes of w (the low pair or the high pair) -> two fp16 in one
// dword. Exact: every e4m3 value (4 significant bits, 2^-9 .. 448) is an
// fp16 value.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi));
}

// two fp32 -> fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const v2h p = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Bias kinds: none, per-head slopes bf16(slope * -d), learned table T[h][min(d, E - 1)].
constexpr int kBiasNone = 0, kBiasSlope = 1, kBiasTable = 2;

// Lazy-rescale slack of the fp8-P variant, log2 units: with P = 2^(x - m + 8)
// and x <= m + slack, P stays below 2^8.75 < 448 (the pages' 0.75, under
// the invariant log2(448) - 8 = 0.807).
constexpr float kLazySlack = 0.75f;

// Lazy-rescale slack of the fp16-P path (P <= 2^8).
constexpr float kLazyF16 = 8.0f;

// P representations of PV: fp16 (default), one e4m3 term, two e4m3 terms.
constexpr int kPF16 = 0, kPFp8 = 1, kPFp8x2 = 2;

// The exponent gap below the running max past which every P is exactly zero:
// fp16 P = 2^(x - m) rounds to 0 below 2^-25 (half the smallest subnormal;
// 2^-25 itself is a tie that goes to the even zero); e4m3 P = 2^(x - m + 8)
// below 2^-10, and its second term, e4m3 of what the first left, is then
// e4m3 of the same value. One more unit keeps the decision clear of the
// rounding of x - m and of exp2's last bit.
template <int kPMode>
constexpr float zero_gap() { return kPMode == kPF16 ? 26.0f : 19.0f; }

template <int kKind, int kPMode>
__global__ __launch_bounds__(64 * kPW) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_e4m3_kernel(PrefillE4M3Launch a, int groups, int units, int head_blocks, int chunk, int nchunks,
                         int tpw) {
  constexpr bool kP8 = kPMode != kPF16;
  constexpr float kGap = zero_gap<kPMode>();
  __shared__ PrefillSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15;
  const int grp = lane >> 4;

  // ---- work item (workgroup i runs on XCD i % 8). A workgroup takes tpw
  // consecutive 32-token tiles (a tile group) of kPW / tpw query heads of one
  // KV head: wave w has head (w % hpw) of its head block and tile (w / hpw)
  // of its group. The tile groups of a unit (sequence, KV head, head block)
  // form nchunks chunks of `chunk` groups; (unit, chunk) pairs go round-robin
  // over the XCDs, so with 8 or more groups every XCD holds one chunk of
  // every unit (the same mix of units, whatever their cost), and each chunk's
  // groups stream the unit's K/V through one L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int pair = (slot / chunk) * 8 + xcd;
  const int u = pair / nchunks;
  const int tg = (pair - u * nchunks) * chunk + slot % chunk;
  if (u >= units || tg >= groups) return;
  const int hpw = kPW / tpw;   // query heads per workgroup
  // Units are numbered KV head outermost, the last KV head first: under the
  // slope bias of the ALiBi family the slopes fall with the head index, so
  // the last heads reach farthest back before their probabilities vanish and
  // cost the most; dispatching them first leaves the cheap units for the end
  // (otherwise the last costly workgroups started late set the kernel's end).
  // Without a slope bias every unit costs about the same and the order does
  // not matter. Within a KV head the head blocks also run last first, and
  // the sequences are innermost: units of one head come together, so
  // consecutive workgroups cost about the same. (Each XCD hands its
  // workgroups to its shader engines in turn and in order; runs of equal
  // cost keep one engine's long workgroups from holding back the dispatch
  // of the next ones while other engines sit idle.)
  const int b = u % a.batch;
  const int hb = head_blocks - 1 - (u / a.batch) % head_blocks;
  const int g = a.hkv - 1 - u / (head_blocks * a.batch);
  const int q0 = a.cu_q_lens[b];
  const int lq = a.cu_q_lens[b + 1] - q0;
  const int tile0 = tg * tpw;                     // the group's first tile
  if (tile0 * kTileTok >= lq) return;
  const int L = a.seq_lens[b];
  const int tile = tile0 + wave / hpw;            // this wave's tile
  const int ntok = max(0, min(kTileTok, lq - tile * kTileTok));   // 0: the wave has no query
  const int P0 = L - lq + tile * kTileTok;        // position of the tile's first token
  const int group = a.hq / a.hkv;
  const int hloc = hb * hpw + wave % hpw;
  const bool head_ok = hloc < group;
  const int head = g * group + (head_ok ? hloc : 0);

  // keys of the workgroup [klo, khi): the union of its rows' ranges (its
  // tokens end at the sequence end at the latest); of this wave [wklo, wkhi)
  const int P0g = L - lq + tile0 * kTileTok;
  const int khi = min(P0g + tpw * kTileTok, L);
  const int klo = a.window > 0 ? max(0, P0g - a.window + 1) : 0;
  const int wkhi = P0 + ntok;
  const int wklo = a.window > 0 ? max(0, P0 - a.window + 1) : 0;
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
  constexpr bool kBias = kKind != kBiasNone;
  const float slope = kKind == kBiasSlope ? a.slopes[head] : 0.0f;
  // slope bias: per row, 448 * sum |q| bounds |q . k| in code units (the
  // margin covers the fp32 sum and the MFMA's accumulation)
  if constexpr (kKind == kBiasSlope) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float acc = 0.0f, acc2 = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(qop[cb][c], false);
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(qop[cb][c], true);
        acc += (fabsf(lo.x) + fabsf(lo.y)) + (fabsf(hi.x) + fabsf(hi.y));
        acc2 += (lo.x * lo.x + lo.y * lo.y) + (hi.x * hi.x + hi.y * hi.y);
      }
      acc += __shfl_xor(acc, 16, 64);
      acc += __shfl_xor(acc, 32, 64);
      acc2 += __shfl_xor(acc2, 16, 64);
      acc2 += __shfl_xor(acc2, 32, 64);
      if (grp == 0) {
        sm.qbound[wave][cb * 16 + row] = acc * (448.0f * 1.001f);
        sm.qnorm[wave][cb * 16 + row] = sqrtf(acc2) * 1.001f;
      }
    }
    // read back by every lane group of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // Slope bias with key norms: pm[i] = the largest key-code norm of blocks
  // blk_lo .. blk_lo + i (an inclusive prefix max: thread t takes blocks 2t
  // and 2t + 1, a wave scan, then the maxima of the earlier waves). A wave at
  // block blk then bounds every remaining raw score of row r by
  // |q_r| * pm[blk - blk_lo] (Cauchy-Schwarz over the codes).
  const bool use_pm = kKind == kBiasSlope && a.knorm != nullptr && blk_lo <= blk_hi &&
                      blk_hi - blk_lo + 1 <= kMaxPM && blk_hi < a.knorm_blocks;
  if (use_pm) {   // uniform over the workgroup
    const float *kn = a.knorm + ((size_t)b * a.hkv + g) * a.knorm_blocks + blk_lo;
    const int n = blk_hi - blk_lo + 1;
    const float v0 = 2 * tid < n ? kn[2 * tid] : 0.0f;
    const float v1 = 2 * tid + 1 < n ? fmaxf(v0, kn[2 * tid + 1]) : v0;
    float x = v1;   // inclusive scan over the wave's lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(x, d, 64);
      if (lane >= d) x = fmaxf(x, y);
    }
    float before = __shfl_up(x, 1, 64);   // lanes below this one
    if (lane == 0) before = 0.0f;
    if (lane == 63) sm.pmw[wave] = x;
    __syncthreads();
    float carry = 0.0f;
    for (int w = 0; w < wave; ++w) carry = fmaxf(carry, sm.pmw[w]);
    if (2 * tid < n) sm.pm[2 * tid] = fmaxf(fmaxf(carry, before), v0);
    if (2 * tid + 1 < n) sm.pm[2 * tid + 1] = fmaxf(carry, x);
    __syncthreads();
  }
  const uint16_t *rel_row = kKind == kBiasTable ? a.rel + (size_t)head * a.rel_extent : nullptr;
  const float rel_last = kKind == kBiasTable ? __uint_as_float((uint32_t)rel_row[a.rel_extent - 1] << 16) * kLog2e : 0.0f;

  float m_run[2] = {-INFINITY, -INFINITY};
  v4f o[2][8];
  v4f ol[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};   // row sums of P (ones tile)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int t = 0; t < 8; ++t) o[cb][t] = v4f{0.f, 0.f, 0.f, 0.f};

  const size_t head_stride = (size_t)16 * kD;
  const size_t page_stride = (size_t)a.hkv * head_stride;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;

  // ---- block loader: thread chunk q in [0, 2048): q < 1024 -> K, else V^T;
  // 128 chunks (2 KB) per page. Pages past the sequence end are clamped.
  // Chunk c of a thread lies in block page (wave / 2) + 4 (c & 1), so a wave
  // needs two page ids per block; they are read two blocks ahead of their
  // load (fetch_ids), which keeps the block-table round trip out of the
  // loads' issue.
  static_assert(kLoadChunks == 4 && 64 * kPW == 512, "chunk -> page mapping");
  uint4 pre[kLoadChunks];
  int ids[2];        // page ids of the next load
  int ids_n[2];      // and of the load after it
  auto fetch_ids = [&](int blk, int (&dst)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) dst[h] = bt[min(blk * 8 + (wave >> 1) + 4 * h, page_last)];
  };
  auto load_block = [&]() {
#pragma unroll
    for (int c = 0; c < kLoadChunks; ++c) {
      const int q = tid + c * 64 * kPW;
      const int tensor = q >> 10;
      const int off = (q & 127) << 4;
      const uint8_t *base = tensor == 0 ? a.kc : a.vc;
      const size_t page_off = (size_t)__builtin_amdgcn_readfirstlane(ids[c & 1]) * page_stride;
      const v4u x = __builtin_nontemporal_load((const v4u *)(base + page_off + (size_t)g * head_stride + off));
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
        sm.k[kidx * 8 + (chunk ^ kswz(kidx))] = pre[c];
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
        const int dim = off >> 4;
        if constexpr (kP8) {
          // e4m3 as stored: the 16 tokens of one dim of one page
          sm.v[pg * 128 + dim] = x;
        } else {
          // tokens 0..7 -> half 0, 8..15 -> half 1, as fp16
          sm.v[(pg * 2 + 0) * 128 + dim] = make_uint4(e4m3x2_to_f16x2<false>(x.x), e4m3x2_to_f16x2<true>(x.x),
                                                       e4m3x2_to_f16x2<false>(x.y), e4m3x2_to_f16x2<true>(x.y));
          sm.v[(pg * 2 + 1) * 128 + dim] = make_uint4(e4m3x2_to_f16x2<false>(x.z), e4m3x2_to_f16x2<true>(x.z),
                                                       e4m3x2_to_f16x2<false>(x.w), e4m3x2_to_f16x2<true>(x.w));
        }
      }
    }
  };

  const float fold = a.fold_log2;
  if (blk_lo <= blk_hi) {   // empty when seq_lens < new tokens
    fetch_ids(blk_hi, ids);
    load_block();
    if (blk_hi > blk_lo) fetch_ids(blk_hi - 1, ids);
  }
  bool wdone = false;   // slope bias: every P of this wave's remaining blocks is zero
  for (int blk = blk_hi; blk >= blk_lo; --blk) {
    const int j0 = blk * kBlkKeys;
    if (blk - 1 > blk_lo) fetch_ids(blk - 2, ids_n);   // page ids of the load after next
    if constexpr (kKind == kBiasSlope) {
      // the remaining keys are <= j0 + 127: the bias of row r is at most the
      // one at distance max(0, P0 + r - (j0 + 127)); rows past the tile's
      // tokens (and waves without a head) are not written and do not count
      if (!wdone && slope >= 0.0f) {
        bool ok = true;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int r = cb * 16 + row;
          const int dmin = max(0, P0 + r - (j0 + kBlkKeys - 1));
          float qk = sm.qbound[wave][r];   // bounds |q . k| over the remaining keys
          if (use_pm) qk = fminf(qk, sm.qnorm[wave][r] * sm.pm[blk - blk_lo]);
          const float ub = fmaf(fold, qk, round_bf16_finite(slope * -(float)dmin) * kLog2e);
          ok = ok && (!head_ok || r >= ntok || ub <= m_run[cb] - kGap);
        }
        wdone = __ballot(!ok) == 0;
      }
      if (lane == 0) sm.done[blk & 1][wave] = wdone ? 1 : 0;
    }
    __syncthreads();                  // everyone is done reading the previous block
    if constexpr (kKind == kBiasSlope) {
      // the eight flags (0 or 1) in two 16-byte reads: a short-circuit loop
      // would wait for each read before issuing the next
      static_assert(kPW == 8, "two uint4 of flags");
      const uint4 f0 = *(const uint4 *)&sm.done[blk & 1][0];
      const uint4 f1 = *(const uint4 *)&sm.done[blk & 1][4];
      if ((f0.x & f0.y & f0.z & f0.w & f1.x & f1.y & f1.z & f1.w) != 0) break;   // uniform
    }
    stash_block(blk);
    __syncthreads();
    if (blk > blk_lo) {
      load_block();
#pragma unroll
      for (int h = 0; h < 2; ++h) ids[h] = ids_n[h];
    }
    if (kKind == kBiasSlope && wdone) continue;
    // a block outside this wave's keys (the workgroup's tiles reach further)
    if (!head_ok || j0 >= wkhi || j0 + kBlkKeys <= wklo) continue;

    const bool edge = (j0 + kBlkKeys - 1 > P0) || (a.window > 0 && j0 < wkhi - a.window);
    // ---- S^T = K Q^T for both column blocks, sharing every K operand read.
    // Lane (row, grp) gets keys kidx = 32*grp + 16*(j/4) + 4*(j%4) + i of
    // query row cb*16 + row.
    v4f s[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kidx = 32 * (row >> 2) + 16 * (j >> 2) + 4 * (j & 3) + (row & 3);
      const int c0 = 2 * grp;
      const uint4 x0 = sm.k[kidx * 8 + (c0 ^ kswz(kidx))];
      const uint4 x1 = sm.k[kidx * 8 + ((c0 + 1) ^ kswz(kidx))];
      const v8i kop = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      s[0][j] = mfma_16x16x128_e4m3(kop, qop[0], v4f{0.f, 0.f, 0.f, 0.f});
      s[1][j] = mfma_16x16x128_e4m3(kop, qop[1], v4f{0.f, 0.f, 0.f, 0.f});
    }
    if constexpr (kKind == kBiasSlope) {
      // Cheap dead-block test: the bias falls with distance, so no exponent
      // argument of row r exceeds fold * (the row's largest raw score) + the
      // bias at the row's nearest key of the block; when that lies kGap or
      // more below the running max in every row of the wave with a query
      // (rows past the tile's tokens are not written), every P of the block
      // is zero: skip it before the bias table and its lookups. (fmaf is
      // monotone in both arguments, so the bound holds after rounding.)
      bool live = false;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float smax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          smax = fmaxf(smax, fmaxf(fmaxf(s[cb][j][0], s[cb][j][1]), fmaxf(s[cb][j][2], s[cb][j][3])));
        smax = wave_max_xor(smax, 16);
        smax = wave_max_xor(smax, 32);
        const int r = cb * 16 + row;
        const int dmin = max(0, P0 + r - (j0 + kBlkKeys - 1));
        const float ub = fmaf(fold, smax, round_bf16_finite(slope * -(float)dmin) * kLog2e);
        live = live || (head_ok && r < ntok && ub > m_run[cb] - kGap);
      }
      if (!__ballot(live)) continue;
    }
    // ---- per-wave bias table for this block: entry e <-> distance
    // d = (P0 - j0) + e - 127, value bf16(slope * -d) or T[min(d, E - 1)],
    // times log2(e). With the learned table, a block whose nearest key is at
    // least E - 1 from the tile's first query reads only the table's last
    // entry (no lookups, no table).
    const bool far = kKind == kBiasTable && P0 - (j0 + kBlkKeys - 1) >= a.rel_extent - 1;
    if (kBias && !far) {
      for (int e = lane; e < kBiasN; e += 64) {
        float val;
        if (kKind == kBiasSlope) {
          const float d = (float)(P0 - j0 + e - 127);
          val = round_bf16_finite(slope * -d) * kLog2e;
        } else {
          const int d = min(max(P0 - j0 + e - 127, 0), a.rel_extent - 1);   // later keys are masked
          val = __uint_as_float((uint32_t)rel_row[d] << 16) * kLog2e;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) sm.bias[wave][bias_copy(g) + e] = val;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    uint4 pk[2][4];     // P in fp16: pk[cb][kk] holds keys 8kk .. 8kk+7 of the lane group
    v8i pk8[2];         // fp8-P variants: byte 4j + i of pk8[cb] is key 32*grp + 4j + i
    v8i pk8l[2];        // two-term variant: the second term, same layout
    const float scale = kBias ? 1.0f : fold;
    float xmax[2];      // the block's largest exponent argument of this lane's query row
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = cb * 16 + row;
      // This lane's keys are j0 + 32*grp + c, c = 16*(j/4) + 4*(j%4) + i in
      // [0, 32). Bias entry r - kidx + 127 = tb_base + (31 - c) with
      // tb_base >= 0, so every lookup is an immediate LDS offset.
      const float *tb = &sm.bias[wave][bias_copy(grp) + r - 32 * grp + 96];
      const int c_hi = P0 + r - j0 - 32 * grp;              // keys with c <= c_hi are causal
      const int c_lo = a.window > 0 ? c_hi - a.window : -1;  // and c > c_lo inside the window
      if (kBias && far) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[cb][j][i] = fmaf(s[cb][j][i], fold, rel_last);
      } else if (kBias) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s[cb][j][i] = fmaf(s[cb][j][i], fold, tb[31 - (16 * (j >> 2) + 4 * (j & 3) + i)]);
      }
      if (edge) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = 16 * (j >> 2) + 4 * (j & 3) + i;
            s[cb][j][i] = (c <= c_hi && c > c_lo) ? s[cb][j][i] : -INFINITY;
          }
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[cb][j][i]);
      bmax = wave_max_xor(bmax, 16);
      bmax = wave_max_xor(bmax, 32);
      xmax[cb] = bmax * scale;
    }
    // Every P of the block is 2^(x - m) (times 2^8 for e4m3 P) with x <= xmax;
    // when xmax lies kGap or more below the running max in every row of the
    // wave, all of them round to zero and PV would add exact zeros: skip the
    // block. (With no key seen yet, m = -inf and a finite xmax is live.)
    if (!__ballot(xmax[0] > m_run[0] - kGap || xmax[1] > m_run[1] - kGap)) continue;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if constexpr (kP8) {
        // single e4m3 term P = 2^(x - m + 8); the running max is raised (to
        // the block max) only when a score passes it by more than the slack
        const bool raise = xmax[cb] > m_run[cb] + kLazySlack;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run[cb] - xmax[cb]) : 1.0f;   // 0 from -inf
        if (raise) m_run[cb] = xmax[cb];
        const float off8 = 8.0f - (m_run[cb] == -INFINITY ? 0.0f : m_run[cb]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(s[cb][j][i], scale, off8));
          const uint32_t hi = cvt4_e4m3(pv[0], pv[1], pv[2], pv[3]);
          pk8[cb][j] = (int)hi;
          if constexpr (kPMode == kPFp8x2) {
            // second term: e4m3 of what the first one left (exact difference
            // in fp32), so each weight keeps about 8 significant bits
            const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
            const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
            pk8l[cb][j] = (int)cvt4_e4m3(pv[0] - h01.x, pv[1] - h01.y, pv[2] - h23.x, pv[3] - h23.y);
          }
        }
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int t = 0; t < 8; ++t) o[cb][t] *= alpha;
          ol[cb] *= alpha;
        }
        continue;
      }
      // lazy max: raised (to the block max) only when a score passes it by
      // more than kLazyF16, so P <= 2^8
      const bool raise = xmax[cb] > m_run[cb] + kLazyF16;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run[cb] - xmax[cb]) : 1.0f;   // 0 from -inf
      if (raise) m_run[cb] = xmax[cb];
      const float m_use = m_run[cb] == -INFINITY ? 0.0f : m_run[cb];
      // P = 2^(x - m); pk[cb][kk] = keys 8kk .. 8kk+7 (j = 2kk, 2kk+1), the
      // B-operand slice of PV step kk
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pv[e] = __builtin_amdgcn_exp2f(fmaf(s[cb][2 * kk + (e >> 2)][e & 3], scale, -m_use));
        pk[cb][kk] = make_uint4(pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]),
                                pack_f16x2(pv[4], pv[5]), pack_f16x2(pv[6], pv[7]));
      }
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) o[cb][t] *= alpha;
        ol[cb] *= alpha;
      }
    }
    if constexpr (kP8) {
      // ---- O^T += V^T P^T on v_mfma_f32_16x16x128_f8f6f4: tile t, dim
      // 16t + row, keys 32*grp .. +32 = the 16 tokens of block pages 2*grp and
      // 2*grp + 1; a ones tile accumulates the row sums of the rounded P
      const v8i ones8 = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                            0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint4 x0 = sm.v[(2 * grp) * 128 + 16 * t + row];
        const uint4 x1 = sm.v[(2 * grp + 1) * 128 + 16 * t + row];
        const v8i va = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        o[0][t] = mfma_16x16x128_e4m3(va, pk8[0], o[0][t]);
        o[1][t] = mfma_16x16x128_e4m3(va, pk8[1], o[1][t]);
        if constexpr (kPMode == kPFp8x2) {
          o[0][t] = mfma_16x16x128_e4m3(va, pk8l[0], o[0][t]);
          o[1][t] = mfma_16x16x128_e4m3(va, pk8l[1], o[1][t]);
        }
      }
      ol[0] = mfma_16x16x128_e4m3(ones8, pk8[0], ol[0]);
      ol[1] = mfma_16x16x128_e4m3(ones8, pk8[1], ol[1]);
      if constexpr (kPMode == kPFp8x2) {
        ol[0] = mfma_16x16x128_e4m3(ones8, pk8l[0], ol[0]);
        ol[1] = mfma_16x16x128_e4m3(ones8, pk8l[1], ol[1]);
      }
      // operands just in time (two LDS reads, then their MFMAs)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, kPMode == kPFp8x2 ? 4 : 2, 0);
      }
      continue;
    }
    // ---- O^T += V^T P^T (fp16 MFMA, 32 keys per step) for both column
    // blocks from one V^T operand read; tile t covers dims 16t .. 16t+15,
    // step kk keys 8kk .. 8kk+7 of every lane group. A ones tile accumulates
    // the row sums of the same rounded P.
    const v8h ones = as_v8h(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const v8h p0 = as_v8h(pk[0][kk]), p1 = as_v8h(pk[1][kk]);
      const uint4 *vrow = sm.v + ((2 * grp + (kk >> 1)) * 2 + (kk & 1)) * 128 + row;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v8h va = as_v8h(vrow[16 * t]);
        o[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, p0, o[0][t], 0, 0, 0);
        o[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, p1, o[1][t], 0, 0, 0);
      }
      ol[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, p0, ol[0], 0, 0, 0);
      ol[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, p1, ol[1], 0, 0, 0);
    }
  }

  // ---- normalise and write bf16 rows: lane holds O[row][16t + 4*grp + i]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = ol[cb][0];
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

// Largest Euclidean norm of the stored key codes of each (sequence, KV head,
// 128-key block), [batch][hkv][nblk]; keys at or past the sequence end do not
// count, blocks past it are not written. One wave per block: load i brings
// keys 8i .. 8i + 7 of the block (page i / 2), lane l chunk l % 8 of key
// 8i + l / 8; the 8 lanes of a key add their squares. The norm is rounded up
// by 1e-4 relative, which covers the fp32 sum of 128 squares (each square of
// an e4m3 code is exact, each addition rounds by at most 2^-24).
constexpr int kNormWaves = 4;
__global__ __launch_bounds__(64 * kNormWaves) void key_norm_kernel(const uint8_t *kc, const int32_t *block_table,
                                                                    int64_t bt_stride, const int32_t *seq_lens,
                                                                    int batch, int hkv, int nblk, float *knorm) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kNormWaves + (int)(threadIdx.x >> 6);   // (b * hkv + g) * nblk + blk
  if (w >= batch * hkv * nblk) return;
  const int blk = w % nblk;
  const int g = (w / nblk) % hkv;
  const int b = w / (nblk * hkv);
  const int L = seq_lens[b];
  if (blk * kBlkKeys >= L) return;
  const int32_t *bt = block_table + (size_t)b * bt_stride;
  const int pid = bt[min(blk * 8 + (lane & 7), (L - 1) >> 4)];
  const size_t head_stride = (size_t)16 * kD;
  const uint8_t *base = kc + (size_t)g * head_stride + (lane >> 3) * kD + 16 * (lane & 7);
  v4u x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const size_t ph = (size_t)__builtin_amdgcn_readlane(pid, i >> 1);
    x[i] = __builtin_nontemporal_load((const v4u *)(base + ph * hkv * head_stride + 8 * (i & 1) * kD));
  }
  float best = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float ss = 0.0f;
    const uint32_t wv[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[c], false);
      const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[c], true);
      ss += (lo.x * lo.x + lo.y * lo.y) + (hi.x * hi.x + hi.y * hi.y);
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    const int pos = blk * kBlkKeys + 8 * i + (lane >> 3);
    if (pos < L) best = fmaxf(best, ss);
  }
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) best = fmaxf(best, __shfl_xor(best, m, 64));
  if (lane == 0) knorm[w] = sqrtf(best) * 1.0001f;
}

}  // namespace

hipError_t launch_prefill_e4m3(const PrefillE4M3Launch &a, hipStream_t s) {
  if (a.d != kD) return hipErrorNotSupported;
  const int group = a.hq / a.hkv;
  const int tiles = (a.max_q_len + kTileTok - 1) / kTileTok;
  if (tiles == 0) return hipSuccess;
  const int kind = a.slopes != nullptr ? kBiasSlope : (a.rel != nullptr ? kBiasTable : kBiasNone);
  // Tiles per workgroup. Under the slope bias each head stops its key walk at
  // its own distance (the smaller the slope, the later), and a workgroup
  // runs until its last wave stops: one head and up to 8 tiles per
  // workgroup keeps all of its waves busy to the end. Otherwise 8 heads of
  // one tile.
  const int tpw = kind != kBiasSlope ? 1 : (tiles >= 8 ? 8 : (tiles >= 4 ? 4 : (tiles >= 2 ? 2 : 1)));
  const int hpw = kPW / tpw;
  const int head_blocks = (group + hpw - 1) / hpw;
  const int units = a.batch * a.hkv * head_blocks;
  const int groups = (tiles + tpw - 1) / tpw;
  const int chunk = groups >= 8 ? (groups + 7) / 8 : groups;   // tile groups per chunk
  const int nchunks = (groups + chunk - 1) / chunk;
  const size_t grid = (size_t)8 * (((size_t)units * nchunks + 7) / 8) * chunk;
  const dim3 g((unsigned)grid), b(64 * kPW);
  PrefillE4M3Launch pa = a;
  // The key-norm pass reads every stored K byte of the batch once, so it runs
  // only when enough query tiles share those bytes (at least 256 new tokens
  // in the longest sequence); shorter calls keep the looser bound.
  if (kind != kBiasSlope || a.max_q_len < 256) pa.knorm = nullptr;
  if (pa.knorm != nullptr) {
    const size_t waves = (size_t)a.batch * a.hkv * a.knorm_blocks;
    hipLaunchKernelGGL(key_norm_kernel, dim3((unsigned)((waves + kNormWaves - 1) / kNormWaves)), dim3(64 * kNormWaves),
                       0, s, a.kc, a.block_table, a.bt_stride, a.seq_lens, a.batch, a.hkv, a.knorm_blocks, a.knorm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define KVQ_PREFILL_LAUNCH(K, P) \
  hipLaunchKernelGGL((prefill_e4m3_kernel<K, P>), g, b, 0, s, pa, groups, units, head_blocks, chunk, nchunks, tpw)
#define KVQ_PREFILL_KINDS(P)                                   \
  do {                                                         \
    if (kind == kBiasSlope) KVQ_PREFILL_LAUNCH(kBiasSlope, P); \
    else if (kind == kBiasTable) KVQ_PREFILL_LAUNCH(kBiasTable, P); \
    else KVQ_PREFILL_LAUNCH(kBiasNone, P);                      \
  } while (0)
  if (a.p_mode == 1) KVQ_PREFILL_KINDS(kPFp8);
  else if (a.p_mode == 2) KVQ_PREFILL_KINDS(kPFp8x2);
  else KVQ_PREFILL_KINDS(kPF16);
#undef KVQ_PREFILL_KINDS
#undef KVQ_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace kvq
