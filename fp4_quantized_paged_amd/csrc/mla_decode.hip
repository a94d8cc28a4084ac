// NVFP4 MLA decode: attention of 16 query heads over one latent KV head
// stored as 368-byte NVFP4 records.
//
// local-inference-lab/vllm PR 189, "mla: wire dynamic per-token NVFP4 scaling
// and cache ABI" (commit message, "Why"): readers take the per-token outer
// scale from bytes [292, 296) of each record instead of a per-layer launch
// scalar. Per key j:
//   latent_j = e2m1(v) * e4m3(sg) * s2_j
//   K_j = [latent_j ; e4m3(rope_j) * rope_scale],  V_j = latent_j
//   s_j = softmax_scale * (s2_j * (q_lat . Kt_j) + rope_scale * (q_rope . r_j))
// with Kt_j = e2m1 * e4m3(sg); out = sum_j p_j s2_j Kt_j / sum_j p_j.
//
// Kernel design (gfx950, wave64, one workgroup of 4 wave pairs per
// (sequence, split); pairs take interleaved 16-key pages):
//  * the two waves of a pair split the 512 latent dims (256 each) and the 64
//    RoPE dims (32 each). Every product e2m1 * e4m3 is exact in fp16, so the
//    latent is dequantized by the hardware fp4 -> fp16 conversion and one
//    packed fp16 multiply per two values. Q is held in registers as fp16,
//    pre-scaled per head by a power of two that puts its largest element in
//    [2^13, 2^14) (exact for all but elements 2^-31 below the head maximum);
//  * QK^T on v_mfma_f32_16x16x32_f16 (A = 16 keys x 32 dims from registers,
//    B = the 16 heads). The two half-dot-products meet through LDS (a
//    handshake of the pair's two waves per page, no workgroup barrier);
//    both waves then run the same softmax on identical scores;
//  * the dequantized rows also go to LDS (chunk-major, bank-conflict free,
//    two buffers per wave) and PV (v_mfma_f32_16x16x16_f16, A = V^T) reads
//    them back with ds_read_b64_tr_b16, whose 16-lane transpose turns four
//    row segments into one dim x 4 keys operand. The PV of page k-1 is
//    interleaved with the dequant and QK^T of page k, so the vector ALU and
//    the matrix cores work at the same time;
//  * each wave keeps four pages of record bytes in flight, loaded straight
//    into the MFMA operand layout (lane = key, 32 contiguous nibble bytes of
//    its dim slice, the four group scales, eight RoPE codes, and the outer
//    scales of the four keys whose scores the lane holds);
//  * P enters PV in fp16. Per pair, Gs is the largest exponent of the outer
//    scales seen so far; the keys' scales enter P as s2 * 2^-Gs < 1. Per head,
//    the running max m is integer-valued and raised only when a score passes
//    it by more than 8 (log2 units), so 2^(x - m) <= 2^8 and P stays far
//    below the fp16 limit. The accumulator holds
//    O_acc = 2^-Gs sum_j 2^(x_j - m) s2_j Kt_j; it is rescaled (by powers of
//    two) only when m or Gs moves;
//  * pairs merge through LDS; with one split the workgroup writes bf16, else
//    (O, m, l, m + Gs) partials go to the workspace for the split combine.

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kPairs = 4;
constexpr int kWaves = 2 * kPairs;
constexpr int kThreads = 64 * kWaves;
constexpr int kRec = 368;
constexpr int kLat = 512;
constexpr int kHalf = 256;            // latent dims per wave
constexpr int kHeads = 16;
constexpr int kKtBytes = 16 * kHalf * 2;          // fp16 K rows of one page, one wave
constexpr int kStageRowU4 = (kLat + 64) / 8 + 1;  // bf16 Q staging row, uint4 units
constexpr float kTau = 8.0f;                      // lazy-max slack, log2 units
constexpr int kGUnset = -(1 << 20);               // Gs before any nonzero outer scale
constexpr int kSlabRow = kHalf + 4;               // merge slab row (floats, padded)
constexpr int kBtPerThread = 4;                   // block-table entries staged per thread
constexpr int kMaxSplitPages = kBtPerThread * kThreads;   // pages of one split (2,048)
constexpr int kBufs = 4;                          // pages of record bytes in flight per wave (5 or 6: slower)

// LDS: two K-row buffers per wave, then the pair exchange. Before the loop
// the first region holds the staged bf16 Q; after it, the merge slabs.
constexpr int kXchOff = kWaves * 2 * kKtBytes;
constexpr int kXchBytes = kPairs * 2 * 2 * 64 * 16;
constexpr int kSmemBytes = kXchOff + kXchBytes;
static_assert(2 * 2 * kHeads * kSlabRow * 4 <= kXchOff, "merge slabs fit");
static_assert(((kHeads * (kLat + 64) / 8 + kThreads - 1) / kThreads * kThreads / ((kLat + 64) / 8) + 1) *
                  kStageRowU4 * 16 <= kXchOff,
              "staged Q, with the prologue's spill-over rows, fits");

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t h2_bits(v2h x) { return __builtin_bit_cast(uint32_t, x); }

// 8 e2m1 codes (element 2i in the low nibble of byte i) times the group scale
// s (both halves equal): exact fp16
__device__ __forceinline__ uint4 fp4x8_f16(uint32_t w, v2h s) {
  return make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s));
}

// 8 e4m3 codes as exact fp16
__device__ __forceinline__ uint4 e4m3x8_f16(uint2 w) {
  return make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false)),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true)),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false)),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true)));
}

// 8 bf16 (one uint4) times 2^k, rounded to fp16
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 x, int k) {
  uint32_t r[4];
  const uint32_t in[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2h h = {(_Float16)__builtin_ldexpf(bf16lo(in[i]), k), (_Float16)__builtin_ldexpf(bf16hi(in[i]), k)};
    r[i] = h2_bits(h);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }

// One wave's share of a page's record bytes, loaded in the MFMA layout
// (lane = key `row`, dim group `grp`).
struct PageOp {
  v4u nib[2];      // e2m1 codes of dims 64*grp .. +64 of the wave's 256
  uint32_t sc;     // their four group scales
  uint2 rp;        // RoPE codes of dims 32*half + 8*grp .. +8
  float s2k[4];    // outer scales of keys 4*grp + i (this lane's scores)
};

// Spins of a pair wait before the wave gives up (each spin sleeps ~64
// cycles; a normal wait takes a few spins). A wave that gives up marks the
// workgroup and its outputs become NaN instead of the kernel hanging.
constexpr int kSpinLimit = 1 << 22;

__global__ __launch_bounds__(kThreads) void mla_decode_kernel(DecodeMlaLaunch a, int splits, int pages_per_split) {
  __shared__ __align__(16) uint8_t smem[kSmemBytes];
  __shared__ float s_m[kPairs][kHeads], s_l[kPairs][kHeads], s_e[kPairs][kHeads];
  __shared__ int s_k[kHeads];
  __shared__ int s_flag[kPairs][2];                    // pages whose half scores are published
  __shared__ int s_err;                                // a pair wait gave up
  __shared__ int s_bt[kMaxSplitPages];                 // this split's block-table slice

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave >> 1;
  const int half = wave & 1;
  const int row = lane & 15;      // key of the A operand / head of the output
  const int grp = lane >> 4;
  // work item: (sequence b, split); the query is row b
  const int b = blockIdx.x / splits;
  const int split = blockIdx.x - b * splits;
  const int L = a.seq_lens[b];
  const int qrow = b;
  const int npages = (L + 15) >> 4;
  const int p_begin = split * pages_per_split;
  const int p_end = min(npages, p_begin + pages_per_split);
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;
  const int nbt = p_end - p_begin;   // at most kMaxSplitPages
  // Page ids first (clamped indexes keep the loads unconditional): this
  // wave's copy of the split's first 64, and the split's block-table slice
  // (one entry per thread).
  const int btw = bt[p_begin + max(0, min(lane, nbt - 1))];
  int btt[kBtPerThread];
#pragma unroll
  for (int j = 0; j < kBtPerThread; ++j)
    btt[j] = bt[p_begin + max(0, min((int)threadIdx.x + j * kThreads, nbt - 1))];
  __builtin_amdgcn_sched_barrier(0);

  // Operand loads, per lane: key `row` of the page at byte 368*row; the
  // nibbles of dims 256*half + 64*grp .. +64 (32 bytes), their group scales
  // (4 bytes), the RoPE codes of dims 32*half + 8*grp .. +8, and the outer
  // scales of keys 4*grp + i. Every page slot issues the same eight loads,
  // so the wait for one buffer never covers the later buffers' loads in
  // flight. Without a page to fetch they read this sequence's Q block
  // instead (18 KB, read anyway, unused).
  const uint32_t off_nib = row * kRec + 128 * half + 32 * grp;
  const uint32_t off_sc = row * kRec + 256 + 16 * half + 4 * grp;
  const uint32_t off_rp = row * kRec + 304 + 32 * half + 8 * grp;
  const uint32_t off_s2 = 4 * grp * kRec + 292;
  const uint8_t *dummy = (const uint8_t *)(a.q + (size_t)qrow * a.hq * (kLat + 64));
  auto fetch_from = [&](const uint8_t *page, PageOp &r) {
    r.nib[0] = *(const v4u *)(page + off_nib);
    r.nib[1] = *(const v4u *)(page + off_nib + 16);
    r.sc = *(const uint32_t *)(page + off_sc);
    r.rp = *(const uint2 *)(page + off_rp);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.s2k[i] = *(const float *)(page + off_s2 + i * kRec);
  };
  // The first four page slots are requested before the Q work (page ids
  // from the wave's own copy), so that their latency overlaps Q's.
  PageOp bufs[kBufs];
#pragma unroll
  for (int k = 0; k < kBufs; ++k) {
    const int p = p_begin + pair + k * kPairs;
    const int ph = __builtin_amdgcn_readlane(btw, pair + k * kPairs);   // a clamped copy past the split
    fetch_from(p < p_end ? a.records + (size_t)ph * (16 * kRec) : dummy, bufs[k]);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- Q: stage bf16 in LDS, find each head's power-of-two scale k (largest
  // element of head h times 2^k in [2^13, 2^14)), keep this lane's operands
  // (head `row`; latent step c: dims 256*half + 64*grp + 8c; RoPE: dims
  // 512 + 32*half + 8*grp) as fp16 Q * 2^k in registers
  uint4 qop[8], qrope;
  {
    // Q is requested behind the first pages, so both arrive in one round trip
    constexpr int kQU4 = kHeads * (kLat + 64) / 8;
    const uint4 *qsrc = (const uint4 *)(a.q + (size_t)qrow * a.hq * (kLat + 64));
    uint4 qv[(kQU4 + kThreads - 1) / kThreads];
#pragma unroll
    for (int j = 0; j < (kQU4 + kThreads - 1) / kThreads; ++j)
      qv[j] = qsrc[min((int)threadIdx.x + j * kThreads, kQU4 - 1)];
#pragma unroll
    for (int j = 0; j < kBtPerThread; ++j)
      if ((int)threadIdx.x + j * kThreads < nbt) s_bt[threadIdx.x + j * kThreads] = btt[j];
    uint4 *qs = (uint4 *)smem;
    // unconditional stores: entries past Q (rows 16 .. 21) land in K-row
    // buffer space that is cleared below
#pragma unroll
    for (int j = 0; j < (kQU4 + kThreads - 1) / kThreads; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int h = c / ((kLat + 64) / 8);
      qs[h * kStageRowU4 + (c - h * ((kLat + 64) / 8))] = qv[j];
    }
    __syncthreads();
    if (wave == 0) {
      const uint4 *qr = qs + row * kStageRowU4;
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        const uint4 v = qr[18 * grp + i];
        am = max(am, max(max(bf16x2_absmax(v.x), bf16x2_absmax(v.y)), max(bf16x2_absmax(v.z), bf16x2_absmax(v.w))));
      }
      am = max(am, (uint32_t)__shfl_xor((int)am, 16, 64));
      am = max(am, (uint32_t)__shfl_xor((int)am, 32, 64));
      // amax < 2^e  ->  amax * 2^(14 - e) in [2^13, 2^14)
      if (grp == 0) s_k[row] = am == 0 ? 0 : 14 - __builtin_amdgcn_frexp_expf(__uint_as_float(am << 16));
    }
    __syncthreads();
    const uint4 *qr = qs + row * kStageRowU4;
    const int k = s_k[row];
#pragma unroll
    for (int c = 0; c < 8; ++c) qop[c] = bf16x8_to_f16(qr[(kHalf * half + 64 * grp + 8 * c) / 8], k);
    qrope = bf16x8_to_f16(qr[(kLat + 32 * half + 8 * grp) / 8], k);
    __syncthreads();
    // K-row buffers start at zero: the PV of a page slot that holds no page
    // multiplies them by P = 0
    for (int c = threadIdx.x; c < kXchOff / 16; c += kThreads) ((uint4 *)smem)[c] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x < 2 * kPairs) (&s_flag[0][0])[threadIdx.x] = 0;
    if (threadIdx.x == 0) s_err = 0;
    __syncthreads();
  }
  const float c_score = __builtin_ldexpf(a.scale_log2, -s_k[row]);   // undoes 2^k of head `row`
  const float c_rope = a.rope_scale * c_score;

  // per head `row`: running integer max m (log2 units) and this lane's part
  // of the denominator; per pair: the outer-scale exponent Gs. The
  // accumulator holds O_acc = 2^-Gs * sum_j 2^(x_j - m) s2_j Kt_j.
  float m_run = -INFINITY;
  float l_run = 0.0f;
  int Gs = kGUnset;
  v4f o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  v4h pb_prev = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};   // P of the previous page

  // K rows, chunk-major: 16-byte chunk ch (dims 8ch .. 8ch+7 of the wave's
  // 256) of key r sits at 256*ch + 16*(r ^ 8*(ch&1)). Row writes (8 or 16
  // keys of one chunk) cover distinct banks; a transposed read serves 32
  // lanes (keys 0-7 or 8-15 of chunks 2q and 2q+1) per pass, and the XOR
  // puts the odd chunk's half of them in the other 128 bytes, so the pass
  // covers all 64 banks once (XOR 4 had left both chunks' keys on the same
  // 32 banks, a 2-way conflict). Buffer j of the wave is kKtBytes further.
  uint8_t *kt = smem + wave * 2 * kKtBytes;
  uint8_t *wbase_e = kt + 2048 * grp + 16 * row;          // even steps: chunk 8*grp + c
  uint8_t *wbase_o = kt + 2048 * grp + 16 * (row ^ 8);    // odd steps
  // transposed reads: lane s of group grp reads key 4*grp + s/4, dims
  // 16q + 4(s%4) .. +4 = chunk 2q + (s%4)/2, 8-byte half (s%4)&1
  const int rc1 = (row & 3) >> 1;
  const uint8_t *rbase = kt + 256 * rc1 + 16 * ((4 * grp + (row >> 2)) ^ (8 * rc1)) + 8 * (row & 1);
  v4f *xch = (v4f *)(smem + kXchOff) + pair * 2 * 2 * 64;   // [buf][half][lane]

  // Pair handshake: the exchange slots and K-row buffers are the pair's own,
  // so only the two waves of a pair meet per page. Each wave publishes a
  // page counter after its half scores of an active slot and, one step
  // later, waits for its partner's counter of that slot; LDS operations of
  // one wave complete in issue order, so a counter that reads n means the
  // partner's scores of slot n - 1 are in place. Both waves run the same
  // slots and publish slot j before they wait for slot j, so every wait
  // ends. A wave overwrites the exchange slot of j only late in slot j + 2,
  // after waiting (early in slot j + 2) for the partner's counter j + 2,
  // which the partner publishes late in its slot j + 1, after its reads of
  // slot j early in that slot.
  typedef __attribute__((address_space(3))) volatile int lds_int;
  lds_int *my_flag = (lds_int *)&s_flag[pair][half];
  lds_int *their_flag = (lds_int *)&s_flag[pair][half ^ 1];
  auto pair_publish = [&](int n) {
    __asm__ volatile("" ::: "memory");
    if (lane == 0) *my_flag = n;
  };
  bool stuck = false;
  auto pair_wait = [&](int n) {
    for (int spins = 0; *their_flag < n;) {
      if (++spins > kSpinLimit) {
        stuck = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __asm__ volatile("" ::: "memory");
  };
  auto fetch = [&](int p, PageOp &r) {
    fetch_from(p < p_end ? a.records + (size_t)__builtin_amdgcn_readfirstlane(s_bt[p - p_begin]) * (16 * kRec) : dummy,
               r);
  };

  // Softmax of page slot j (page p), one page later than its QK^T: the
  // partner's half scores of slot j were published a whole step earlier, so
  // the wait for them almost never stalls. Sets pb_prev = P of slot j.
  auto softmax_of = [&](int j, int p, const float (&s2p)[4]) {
    const bool tail = (p + 1) * 16 > L;
    pair_wait(j + 1);
    const v4f y0 = xch[(j & 1) * 128 + lane];
    const v4f y1 = xch[(j & 1) * 128 + 64 + lane];
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = y0[i] + y1[i];
    if (tail) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p * 16 + 4 * grp + i >= L) x[i] = -INFINITY;
    }
    bool raise_m = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) raise_m |= x[i] > m_run + kTau;
    if (__ballot(raise_m)) {
      float bmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bmax = xor_max(xor_max(bmax, 16), 32);
      if (bmax > m_run + kTau) {
        const float m_new = __builtin_ceilf(bmax);
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);   // power of two
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
    pb_prev = v4h{(_Float16)pw[0], (_Float16)pw[1], (_Float16)pw[2], (_Float16)pw[3]};
  };

  // Page slot k of this pair (page p = p_begin + pair + k*kPairs, if below
  // p_end): the softmax of slot k-1; dequant + QK^T of page k (bytes in `op`)
  // into K-row buffer k&1, interleaved with the PV of page k-1 from the other
  // buffer; this wave's half scores of page k published for the partner; then
  // `op` is refilled with slot k+kBufs. Slots past p_end come last and
  // publish nothing (neither wave of the pair reads their scores).
  float s2p_prev[4] = {0.f, 0.f, 0.f, 0.f};   // P scales of slot k-1
  auto step = [&](PageOp &op, int k) {
    const int p = p_begin + pair + k * kPairs;
    const bool active = p < p_end;        // uniform over the wave
    const bool tail = (p + 1) * 16 > L;   // the sequence's last, partial page
    const int cb = (k & 1) * kKtBytes;    // this page's K-row buffer
    const int pbuf = kKtBytes - cb;       // the previous page's, and the next's
    pb_prev = v4h{(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
    if (k > 0 && p - kPairs < p_end) softmax_of(k - 1, p - kPairs, s2p_prev);
    // Keys past the end, and every key of a slot without a page: group
    // scales (possibly NaN codes) and outer scales become zero, so their K
    // rows, V rows and P entries are exactly zero; their scores are masked.
    if (!active || tail) {
      if (!active || p * 16 + row >= L) op.sc = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!active || p * 16 + 4 * grp + i >= L) op.s2k[i] = 0.0f;
    }
    // ---- outer-scale exponent of the pair (both waves see the same keys);
    // a raise rescales the accumulator after the previous page's PV
    const float s2max = fmaxf(fmaxf(op.s2k[0], op.s2k[1]), fmaxf(op.s2k[2], op.s2k[3]));
    const int e2 = __builtin_amdgcn_frexp_expf(s2max);
    int g_new = Gs;
    if (__ballot(s2max > 0.0f && e2 > Gs)) {
      int emax = s2max > 0.0f ? e2 : kGUnset;
      emax = max(emax, __shfl_xor(emax, 16, 64));
      emax = max(emax, __shfl_xor(emax, 32, 64));
      g_new = __builtin_amdgcn_readfirstlane(emax);
    }
    // ---- dequant + QK^T of this page, PV of the previous page
    const v2h sg01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(op.sc, 1.0f, false);
    const v2h sg23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(op.sc, 1.0f, true);
    v4f acc_l = v4f{0.f, 0.f, 0.f, 0.f};
    // PV operand reads run kLook tiles ahead of their MFMAs (2, 8 and 16
    // measured within 1% of each other)
    constexpr int kLook = 8;
    v4s va[16];
    auto read_tile = [&](int q) {
      va[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(rbase + pbuf + 512 * q));
    };
#pragma unroll
    for (int q = 0; q < kLook; ++q) read_tile(q);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (2 * c + j + kLook < 16) read_tile(2 * c + j + kLook);
      const _Float16 s = (c >> 2) == 0 ? sg01[(c >> 1) & 1] : sg23[(c >> 1) & 1];
      const uint4 x = fp4x8_f16(op.nib[c >> 2][c & 3], v2h{s, s});
      *(uint4 *)(((c & 1) ? wbase_o : wbase_e) + cb + 256 * c) = x;
      acc_l = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x), __builtin_bit_cast(v8h, qop[c]),
                                                     acc_l, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = 2 * c + j;   // PV tile: dims 16q .. 16q+15
        o[q] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, va[q]), pb_prev, o[q], 0, 0, 0);
      }
    }
    const uint4 xr = e4m3x8_f16(op.rp);
    const v4f acc_r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xr), __builtin_bit_cast(v8h, qrope),
                                                             v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    if (g_new != Gs) {
      const float f = __builtin_ldexpf(1.0f, max(Gs - g_new, -200));
#pragma unroll
      for (int q = 0; q < 16; ++q) o[q] *= f;
      Gs = g_new;
    }
    // this wave's part of the log2-domain scores of keys 4*grp + i, head `row`
    if (active) {
      v4f y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = fmaf(c_score * op.s2k[i], acc_l[i], c_rope * acc_r[i]);
        s2p_prev[i] = __builtin_ldexpf(op.s2k[i], -Gs);   // < 1
      }
      xch[(k & 1) * 128 + half * 64 + lane] = y;
      pair_publish(k + 1);
    }
    // ---- this load buffer's next slot
    fetch(p + kBufs * kPairs, op);
  };

  const int iters = p_end > p_begin ? (p_end - p_begin + kPairs - 1) / kPairs : 0;
  // slot k sits in load buffer k % kBufs
  int it = 0;
  for (; it + kBufs - 1 < iters; it += kBufs) {
#pragma unroll
    for (int j = 0; j < kBufs; ++j) step(bufs[j], it + j);
  }
#pragma unroll
  for (int j = 0; j < kBufs - 1; ++j)
    if (it + j < iters) step(bufs[j], it + j);
  // softmax and PV of the last page slot (K-row buffer (iters - 1) & 1; P is
  // zero if that slot held no page or there was none)
  {
    pb_prev = v4h{(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
    const int p_last = p_begin + pair + (iters - 1) * kPairs;
    if (iters > 0 && p_last < p_end) softmax_of(iters - 1, p_last, s2p_prev);
    const int pbuf = ((iters - 1) & 1) * kKtBytes;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const v4s va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s *)(rbase + pbuf + 512 * q));
      o[q] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, va), pb_prev, o[q], 0, 0, 0);
    }
  }

  // ---- merge the pairs. Pair totals per head: l_abs = 2^m l,
  // O_abs = 2^(m + Gs) O_acc.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const bool has_o = m_run != -INFINITY && Gs != kGUnset;
  const float my_e = has_o ? m_run + (float)Gs : -INFINITY;
  if (stuck) s_err = 1;
  if (half == 0 && grp == 0) {
    s_m[pair][row] = m_run;
    s_l[pair][row] = l_run;
    s_e[pair][row] = my_e;
  }
  __syncthreads();   // also: every wave is past its last K-row read
  float E = -INFINITY;
#pragma unroll
  for (int q = 0; q < kPairs; ++q) E = fmaxf(E, s_e[q][row]);
  {
    const float f = my_e == -INFINITY ? 0.0f : __builtin_ldexpf(1.0f, max((int)(my_e - E), -200));
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q] *= f;
  }
  // pairs 2, 3 hand their halves to pairs 0, 1, which add them in place; the
  // last add happens on the way out
  float *slab = (float *)smem;   // [2 pair slots][2 halves][16 heads][kSlabRow]
  auto slab_at = [&](int slot, int h, int hd, int d) -> float * {
    return slab + ((size_t)(slot * 2 + h) * kHeads + hd) * kSlabRow + d;
  };
  if (pair >= 2) {
#pragma unroll
    for (int q = 0; q < 16; ++q) *(v4f *)slab_at(pair - 2, half, row, 16 * q + 4 * grp) = o[q];
  }
  __syncthreads();
  if (pair < 2) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      v4f *dst = (v4f *)slab_at(pair, half, row, 16 * q + 4 * grp);
      *dst = o[q] + *dst;
    }
  }
  __syncthreads();
  // a pair wait that gave up leaves NaN outputs (or NaN partials, which the
  // combine turns into NaN outputs) rather than silently wrong values
  const bool failed = s_err != 0;
  // output: 4 consecutive dims per thread and pass
  for (int e4 = threadIdx.x; e4 < kHeads * kLat / 4; e4 += kThreads) {
    const int hd = e4 / (kLat / 4);
    const int d = 4 * (e4 - hd * (kLat / 4));
    const int h = d / kHalf;
    const int dd = d - h * kHalf;
    const v4f acc = *(const v4f *)slab_at(0, h, hd, dd) + *(const v4f *)slab_at(1, h, hd, dd);
    float Mh = -INFINITY, Eh = -INFINITY, den = 0.0f;
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      Mh = fmaxf(Mh, s_m[q][hd]);
      Eh = fmaxf(Eh, s_e[q][hd]);
    }
    if (Mh != -INFINITY) {
#pragma unroll
      for (int q = 0; q < kPairs; ++q)
        if (s_m[q][hd] != -INFINITY) den += __builtin_amdgcn_exp2f(s_m[q][hd] - Mh) * s_l[q][hd];
    }
    if (splits == 1) {
      float sc = 0.0f;
      if (den > 0.0f && Eh != -INFINITY) sc = __builtin_ldexpf(1.0f / den, (int)(Eh - Mh));
      uint2 w;
      w.x = f32_to_bf16_bits(acc[0] * sc) | (f32_to_bf16_bits(acc[1] * sc) << 16);
      w.y = f32_to_bf16_bits(acc[2] * sc) | (f32_to_bf16_bits(acc[3] * sc) << 16);
      if (failed) w = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
      *(uint2 *)(a.out + ((size_t)qrow * a.hq + hd) * kLat + d) = w;
    } else {
      const size_t pi = ((size_t)b * a.hq + hd) * splits + split;
      *(v4f *)(a.part_o + pi * kLat + d) = failed ? v4f{NAN, NAN, NAN, NAN} : acc;
      if (d == 0) *(v4f *)(a.part_ml + 4 * pi) = v4f{Mh, den, Eh, 0.0f};
    }
  }
}

// Split combine: per (sequence, head), out = 2^(E - M) * sum_s 2^(E_s - E) O_s
// / sum_s 2^(M_s - M) den_s. Splits that saw no key (M_s = -inf, den_s = 0)
// and splits with no nonzero term (E_s = -inf) drop out. One thread per 4
// dims; the first splits' partials are requested with the split statistics.
constexpr int kCombineThreads = kLat / 4;
constexpr int kMaxCombineSplits = 64;
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(const float *part_o, const float *part_ml,
                                                                      uint16_t *out, int splits) {
  __shared__ float s_w[2][kMaxCombineSplits];   // per split: O weight, denominator weight
  __shared__ float s_f;                          // 2^(E - M) / den, or 0
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const float *ml = part_ml + (size_t)bh * splits * 4;
  const float *po = part_o + (size_t)bh * splits * kLat + 4 * t;
  // the first kPre splits' partials are requested together with the split
  // statistics (one memory round trip); clamped copies past the last split
  // are not used
  constexpr int kPre = 8;
  v4f pre[kPre];
#pragma unroll
  for (int s = 0; s < kPre; ++s) pre[s] = *(const v4f *)(po + (size_t)min(s, splits - 1) * kLat);
  if (t < 64) {
    float M = -INFINITY, E = -INFINITY;
    const v4f r = t < splits ? *(const v4f *)(ml + 4 * t) : v4f{-INFINITY, 0.f, -INFINITY, 0.f};
    M = r[0];
    E = r[2];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      M = fmaxf(M, __shfl_xor(M, m, 64));
      E = fmaxf(E, __shfl_xor(E, m, 64));
    }
    float wd = 0.0f, wo = 0.0f;
    if (t < splits) {
      if (r[0] != -INFINITY) wd = __builtin_amdgcn_exp2f(r[0] - M) * r[1];
      if (r[2] != -INFINITY) wo = __builtin_ldexpf(1.0f, max((int)(r[2] - E), -200));
      s_w[0][t] = wo;
    }
    float den = wd;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m, 64);
    if (t == 0) s_f = (den > 0.0f && E != -INFINITY) ? __builtin_ldexpf(1.0f / den, (int)(E - M)) : 0.0f;
  }
  __syncthreads();
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < splits) acc += s_w[0][s] * pre[s];
  for (int s = kPre; s < splits; ++s) acc += s_w[0][s] * *(const v4f *)(po + (size_t)s * kLat);
  const float f = s_f;
  uint2 w;
  w.x = f32_to_bf16_bits(acc[0] * f) | (f32_to_bf16_bits(acc[1] * f) << 16);
  w.y = f32_to_bf16_bits(acc[2] * f) | (f32_to_bf16_bits(acc[3] * f) << 16);
  *(uint2 *)(out + (size_t)bh * kLat + 4 * t) = w;
}

}  // namespace

hipError_t launch_decode_mla(const DecodeMlaLaunch &a, const MlaPlan &p, hipStream_t s) {
  if (a.hq != kHeads) return hipErrorNotSupported;
  hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)((size_t)a.batch * p.splits)), dim3(kThreads), 0, s, a,
                     p.splits, p.pages_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((size_t)a.batch * a.hq)), dim3(kCombineThreads), 0, s,
                     a.part_o, a.part_ml, a.out, p.splits);
  return hipGetLastError();
}

}  // namespace kvq
