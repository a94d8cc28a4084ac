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
// (sequence, split); each step of the workgroup covers 8 consecutive pages,
// two per pair, one per wave):
//  * every wave computes the whole QK^T and the softmax of its own page: the
//    latent is dequantized by the hardware fp4 -> fp16 conversion and one
//    packed fp16 multiply per two values (every e2m1 * e4m3 product is exact
//    in fp16), and v_mfma_f32_16x16x32_f16 takes A = 16 keys x 32 dims from
//    registers and B = the 16 heads' Q (fp16, pre-scaled per head by the power
//    of two that puts its largest element in [2^13, 2^14); exact for all but
//    elements 2^-31 below the head maximum);
//  * the dequantized rows also go to LDS (16 KB per wave, chunk-major and
//    bank-conflict free); once the partner's counter shows its rows and P of
//    the step in place, each wave of a pair takes half of the 512 latent dims
//    of PV over both of the pair's pages: v_mfma_f32_16x16x32_f16 with
//    A = V^T (two ds_read_b64_tr_b16 16-lane transposes, four keys of each
//    page) and B = the two pages' P, which the pair exchanges through LDS in
//    fp16. The partner's next counter value tells a wave that its rows have
//    been read before it overwrites them (no workgroup barrier in the page
//    loop; the waits are bounded, and a wave that gives up turns the
//    workgroup's outputs into NaN instead of hanging);
//  * P enters PV in fp16 as 2^(x - m) * s2 * 2^-Gs. Per pair and head, the
//    running max m is integer-valued and raised only when a score passes it
//    by more than 8 (log2 units); Gs is the largest exponent of the outer
//    scales seen, so P <= 2^8 and s2 * 2^-Gs < 1. Each wave raises m and Gs
//    for its own page; after the exchange both waves take the larger values
//    and rescale by powers of two (the accumulator, the denominator, and each
//    page's P), so both halves of the pair hold the same m and Gs;
//  * each wave keeps the record bytes of its next two pages in flight,
//    loaded straight into the operand layout (lane = key, 64 contiguous
//    nibble bytes, their 8 group scales, 16 RoPE codes, and the outer scales
//    of the four keys whose scores the lane holds);
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
constexpr int kHalf = 256;                        // latent dims of PV per wave
constexpr int kHeads = 16;
constexpr int kRowBytes = 16 * kLat * 2;          // fp16 latent rows of one page
constexpr int kStageRowU4 = (kLat + 64) / 8 + 1;  // bf16 Q staging row, uint4 units
constexpr float kTau = 8.0f;                      // lazy-max slack, log2 units
constexpr int kGUnset = -(1 << 20);               // Gs before any nonzero outer scale
constexpr int kBtPerThread = 4;                   // block-table entries staged per thread
constexpr int kMaxSplitPages = kBtPerThread * kThreads;   // pages of one split (2,048)
constexpr int kBufs = 2;                          // pages of record bytes in flight per wave
constexpr int kStepPages = kWaves;                // pages per workgroup step
// Spins of a pair wait before the wave gives up (each spin sleeps ~64
// cycles; a normal wait takes a few spins).
constexpr int kSpinLimit = 1 << 22;
constexpr int kQReg = 16;                         // latent QK^T steps whose Q operand stays in registers
constexpr int kQLds = 16 + 2 - kQReg;             // the other latent steps and the 2 RoPE steps: from LDS

// LDS: the latent rows of each wave's page. Before the loop the region holds
// the staged bf16 Q; after it, the merge slabs.
constexpr int kRowsBytes = kWaves * kRowBytes;
static_assert(kWaves * 16 * 64 * 16 <= kRowsBytes, "merge slabs fit");
static_assert(((kHeads * (kLat + 64) / 8 + kThreads - 1) / kThreads * kThreads / ((kLat + 64) / 8) + 1) *
                  kStageRowU4 * 16 <= kRowsBytes,
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

// 2^e as fp32 for an integer-valued e (0 below 2^-200)
__device__ __forceinline__ float pow2i(float e) { return __builtin_ldexpf(1.0f, max((int)e, -200)); }

// Block i of a grid of batch * inner blocks -> (sequence b, inner index j).
// Workgroups are dispatched to the 8 XCDs round robin (block i on XCD i % 8);
// when batch is a multiple of 8 every block of sequence b lands on XCD b % 8,
// so the split partials of a sequence stay in one XCD's L2 for the combine.
__device__ __forceinline__ void xcd_local(int i, int batch, int inner, int &b, int &j) {
  if ((batch & 7) == 0) {
    const int nb = batch >> 3;
    const int r = i >> 3;
    b = (r % nb) * 8 + (i & 7);
    j = r / nb;
  } else {
    b = i / inner;
    j = i - b * inner;
  }
}

// The record bytes of one page that a wave needs, in the MFMA layout (lane =
// key `row`, dim group `grp`).
struct PageOp {
  v4u nib[4];      // e2m1 codes of latent dims 128*grp .. +128
  uint2 sc;        // their 8 group scales
  v4u rp;          // RoPE codes of dims 16*grp .. +16
  float s2;        // outer scale of key 4*grp + row%4 (its quad holds keys 4*grp .. +4)
};

__global__ __launch_bounds__(kThreads) void mla_decode_kernel(DecodeMlaLaunch a, int splits, int pages_per_split) {
  __shared__ __align__(16) uint8_t smem[kRowsBytes];
  __shared__ uint2 s_p[kWaves][64];                   // each wave's P of its page (fp16 x 4 per lane)
  __shared__ float s_mp[kWaves][kHeads];              // the m that P was taken against
  __shared__ int s_gp[kWaves];                        // the Gs that P was taken against
  __shared__ float s_m[kPairs][kHeads], s_e[kPairs][kHeads], s_l[kWaves][kHeads];
  __shared__ int s_k[kHeads];
  __shared__ v4f s_hf[kHeads];                        // per head: output scale, or (M, den, E) of the split
  __shared__ int s_flag[kWaves];                      // pair handshake counters
  __shared__ int s_err;                               // a pair wait gave up
  __shared__ int s_bt[kMaxSplitPages];                // this split's block-table slice
  __shared__ uint4 s_q[kQLds][64];                    // fp16 Q operands of steps kQReg .. 17, per lane

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the two waves of a pair are neighbours (different SIMDs); every SIMD
  // carries waves of two pairs, which need not be in the same phase
  const int pair = wave >> 1;
  const int half = wave & 1;
  const int partner = wave ^ 1;
  const int wpos = 2 * pair + half;   // this wave's page within a step
  const int row = lane & 15;          // key of the A operand / head of the output
  const int grp = lane >> 4;
  // work item: (sequence b, split); the query is row b
  int b, split;
  xcd_local(blockIdx.x, a.batch, splits, b, split);
  const int qrow = b;
  const int p_begin = split * pages_per_split;
  const int32_t *bt = a.block_table + (size_t)b * a.bt_stride;
  const int bt_last = (int)a.bt_stride - 1;
  // Sequence length, page ids and Q are requested together: the block-table
  // reads are clamped to the table row, not to the sequence, so they need no
  // length (entries past the sequence are never used as addresses).
  const int L = a.seq_lens[b];
  const int btw = bt[min(p_begin + lane, bt_last)];
  int btt[kBtPerThread];
#pragma unroll
  for (int j = 0; j < kBtPerThread; ++j) btt[j] = bt[min(p_begin + (int)threadIdx.x + j * kThreads, bt_last)];
  constexpr int kQU4 = kHeads * (kLat + 64) / 8;
  constexpr int kQPer = (kQU4 + kThreads - 1) / kThreads;
  const uint4 *qsrc = (const uint4 *)(a.q + (size_t)qrow * a.hq * (kLat + 64));
  uint4 qv[kQPer];
#pragma unroll
  for (int j = 0; j < kQPer; ++j) qv[j] = qsrc[min((int)threadIdx.x + j * kThreads, kQU4 - 1)];
  const int npages = (L + 15) >> 4;
  const int p_end = min(npages, p_begin + pages_per_split);
  const int nsteps = p_end > p_begin ? (p_end - p_begin + kStepPages - 1) / kStepPages : 0;

  // Operand loads, per lane: key `row` of the page at byte 368*row; the
  // nibbles of latent dims 128*grp .. +128 (64 bytes), their 8 group scales,
  // the RoPE codes of dims 16*grp .. +16, and the outer scale of key
  // 4*grp + row%4 (a quad broadcast gives each lane the outer scales of the
  // four keys whose scores it holds). Raw buffer loads: the page address sits
  // in the scalar resource and each lane adds its constant 32-bit offset; a
  // slot without a page gets a resource of zero bytes, whose loads return 0.
  const uint32_t off_nib = row * kRec + 64 * grp;
  const uint32_t off_sc = row * kRec + 256 + 8 * grp;
  const uint32_t off_rp = row * kRec + 304 + 16 * grp;
  const uint32_t off_s2 = (4 * grp + (row & 3)) * kRec + 292;
  auto fetch_page = [&](bool act, int ph, PageOp &r) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.records + (size_t)(act ? ph : 0) * (16 * kRec)), (short)0, act ? 16 * kRec : 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.nib[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off_nib + 16 * i, 0, 0);
    r.sc = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off_sc, 0, 0));
    r.rp = __builtin_amdgcn_raw_buffer_load_b128(rs, off_rp, 0, 0);
    r.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off_s2, 0, 0));
  };
  PageOp bufs[kBufs];

  // ---- Q: stage bf16 in LDS, find each head's power-of-two scale k (largest
  // element of head h times 2^k in [2^13, 2^14)), and form this lane's
  // operands (head `row`; latent step c: dims 128*grp + 8c; RoPE step u:
  // dims 512 + 16*grp + 8u) as fp16 Q * 2^k: the first kQReg latent steps in
  // registers, the rest in LDS (the same for every wave, written once)
  uint4 qop[kQReg];
  {
#pragma unroll
    for (int j = 0; j < kBtPerThread; ++j) s_bt[threadIdx.x + j * kThreads] = btt[j];
    if (threadIdx.x < kWaves) s_flag[threadIdx.x] = 0;
    if (threadIdx.x == 0) s_err = 0;
    uint4 *qs = (uint4 *)smem;
    // unconditional stores: entries past Q (rows 16 .. 21) land in row space
    // that is overwritten before it is read
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int h = c / ((kLat + 64) / 8);
      qs[h * kStageRowU4 + (c - h * ((kLat + 64) / 8))] = qv[j];
    }
    __syncthreads();
    // the first pages' record bytes, requested once Q is staged (the loads
    // of Q are then not waited for together with them)
#pragma unroll
    for (int k = 0; k < kBufs; ++k) {
      const int p = p_begin + kStepPages * k + wpos;
      fetch_page(p < p_end, __builtin_amdgcn_readlane(btw, kStepPages * k + wpos), bufs[k]);
    }
    __builtin_amdgcn_sched_barrier(0);
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
    for (int c = 0; c < kQReg; ++c) qop[c] = bf16x8_to_f16(qr[16 * grp + c], k);
    for (int j = wave; j < kQLds; j += kWaves) {
      const int c = kQReg + j;
      s_q[j][lane] = bf16x8_to_f16(qr[c < 16 ? 16 * grp + c : (kLat + 16 * grp + 8 * (c - 16)) / 8], k);
    }
  }
  __syncthreads();   // staged Q read, s_q written, flags cleared: rows may be written
  const float c_score = __builtin_ldexpf(a.scale_log2, -s_k[row]);   // undoes 2^k of head `row`
  const float c_rope = a.rope_scale * c_score;

  // Pair state, equal in both waves: per head `row` the running integer max
  // m (log2 units); the outer-scale exponent Gs. Per wave: this lane's part
  // of the denominator of the wave's own pages (relative to m). The
  // accumulator holds O_acc = 2^-Gs * sum_j 2^(x_j - m) s2_j Kt_j over the
  // pair's pages, for dims 256*half .. +256.
  float m_run = -INFINITY;
  float l_run = 0.0f;
  int Gs = kGUnset;
  v4f o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // Latent rows, chunk-major: 16-byte chunk ch (dims 8ch .. 8ch+7) of key r
  // sits at 256*ch + 16*(r ^ 8*(ch&1)) of the wave's 16 KB. Row writes (16
  // keys of one chunk) cover distinct banks; a transposed read serves 32
  // lanes (keys 0-7 or 8-15 of chunks 2q and 2q+1) per pass, and the XOR puts
  // the odd chunk's half of them in the other 128 bytes, so the pass covers
  // all 64 banks once.
  uint8_t *myrows = smem + wave * kRowBytes;
  uint8_t *wbase_e = myrows + 4096 * grp + 16 * row;          // even steps c: chunk 16*grp + c
  uint8_t *wbase_o = myrows + 4096 * grp + 16 * (row ^ 8);    // odd steps
  // transposed reads: lane s of group grp reads key 4*grp + s/4, dims
  // 16q + 4(s%4) .. +4 = chunk 2q + (s%4)/2, 8-byte half (s%4)&1; tile q of
  // this wave's dim half is 512*(16*half + q) further
  const int rc1 = (row & 3) >> 1;
  const int rd_off = 256 * rc1 + 16 * ((4 * grp + (row >> 2)) ^ (8 * rc1)) + 8 * (row & 1) + 8192 * half;
  const uint8_t *rd0 = smem + (2 * pair) * kRowBytes + rd_off;       // page of the pair's half-0 wave
  const uint8_t *rd1 = smem + (2 * pair + 1) * kRowBytes + rd_off;   // page of its half-1 wave

  // Pair handshake through LDS counters. Step k: a wave publishes 2k+1 once
  // its rows and P are written, and 2k+2 once its PV has read the partner's
  // rows and P; before writing rows of step k it waits for the partner's 2k,
  // before its PV for the partner's 2k+1. LDS operations of one wave complete
  // in issue order, so a counter read as n means everything the partner
  // wrote before publishing n is in place. Each wait is for a value the
  // partner publishes before its own wait for the same value, so every wait
  // ends; a wave that spins past the limit marks the workgroup (NaN outputs)
  // instead of hanging.
  typedef __attribute__((address_space(3))) volatile int lds_int;
  lds_int *my_flag = (lds_int *)&s_flag[wave];
  lds_int *their_flag = (lds_int *)&s_flag[partner];
  bool stuck = false;
  auto pair_publish = [&](int n) {
    __asm__ volatile("" ::: "memory");
    if (lane == 0) *my_flag = n;
  };
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

  auto fetch = [&](int k, PageOp &r) {
    const int p = p_begin + kStepPages * k + wpos;
    const bool act = p < p_end;
    fetch_page(act, act ? __builtin_amdgcn_readfirstlane(s_bt[p - p_begin]) : 0, r);
  };

  // Step k: page p = p_begin + 8k + wpos of this wave.
  auto step = [&](PageOp &op, int k) {
    // the two waves of a SIMD take turns at the higher issue priority, step
    // by step (the older wave would otherwise always win the arbitration)
    if (((k + (wave >> 2)) & 1) != 0) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    const int p = p_begin + kStepPages * k + wpos;
    // a page past the split, or the sequence's last, partial page: some or
    // all keys masked (uniform over the wave)
    const bool tail = p >= p_end || (p + 1) * 16 > L;
    const int kend = p < p_end ? L - p * 16 : 0;   // keys of the page that exist
    // Keys past the end, and every key of a slot without a page: group
    // scales (possibly NaN codes) and outer scales become zero, so their rows
    // and P entries are exactly zero; their scores are masked.
    // outer scales of keys 4*grp + i: quad_perm broadcasts of lane i of the quad
    const int s2b = __builtin_bit_cast(int, op.s2);
    float s2k[4] = {__builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(s2b, 0x00, 0xF, 0xF, false)),
                    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(s2b, 0x55, 0xF, 0xF, false)),
                    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(s2b, 0xAA, 0xF, 0xF, false)),
                    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(s2b, 0xFF, 0xF, 0xF, false))};
    if (tail) {
      if (row >= kend) op.sc = make_uint2(0u, 0u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * grp + i >= kend) s2k[i] = 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
    pair_wait(2 * k);   // the partner's PV of the previous step has read these rows
    __builtin_amdgcn_sched_barrier(0);
    // ---- dequant + rows + QK^T of this wave's page (two accumulators)
    v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = acc0, accr = acc0;
    const v2h sg[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(op.sc.x, 1.0f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(op.sc.x, 1.0f, true),
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(op.sc.y, 1.0f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(op.sc.y, 1.0f, true)};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const _Float16 s = sg[c >> 2][(c >> 1) & 1];   // group 8*grp + c/2
      const uint4 x = fp4x8_f16(op.nib[c >> 2][c & 3], v2h{s, s});
      *(uint4 *)(((c & 1) ? wbase_o : wbase_e) + 256 * c) = x;
      const uint4 qc = c < kQReg ? qop[c < kQReg ? c : 0] : s_q[c < kQReg ? 0 : c - kQReg][lane];
      if (c & 1)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x), __builtin_bit_cast(v8h, qc), acc1,
                                                      0, 0, 0);
      else
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x), __builtin_bit_cast(v8h, qc), acc0,
                                                      0, 0, 0);
      // one step's dequant in registers at a time (the scheduler would
      // otherwise batch them)
      if (c & 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 xr = e4m3x8_f16(u == 0 ? make_uint2(op.rp.x, op.rp.y) : make_uint2(op.rp.z, op.rp.w));
      accr = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xr),
                                                    __builtin_bit_cast(v8h, s_q[16 - kQReg + u][lane]), accr, 0, 0, 0);
    }
    // ---- log2-domain scores of keys 4*grp + i, head `row`; softmax of the
    // page against the pair's m and Gs, raised for this page if needed
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = fmaf(c_score * s2k[i], acc0[i] + acc1[i], c_rope * accr[i]);
    if (tail) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * grp + i >= kend) x[i] = -INFINITY;
    }
    float m_self = m_run;
    bool raise_m = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) raise_m |= x[i] > m_run + kTau;
    if (__ballot(raise_m)) {
      float bmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bmax = xor_max(xor_max(bmax, 16), 32);
      if (bmax > m_run + kTau) m_self = __builtin_ceilf(bmax);
    }
    int g_self = Gs;
    {
      const float s2max = fmaxf(fmaxf(s2k[0], s2k[1]), fmaxf(s2k[2], s2k[3]));
      const int e2 = __builtin_amdgcn_frexp_expf(s2max);
      if (__ballot(s2max > 0.0f && e2 > Gs)) {
        int emax = s2max > 0.0f ? e2 : kGUnset;
        emax = max(emax, __shfl_xor(emax, 16, 64));
        emax = max(emax, __shfl_xor(emax, 32, 64));
        g_self = max(Gs, __builtin_amdgcn_readfirstlane(emax));
      }
    }
    float pe[4];
    float psum = 0.0f;
    v4h pw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pe[i] = m_self == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[i] - m_self);   // <= 2^8
      psum += pe[i];
      pw[i] = (_Float16)(pe[i] * __builtin_ldexpf(s2k[i], -g_self));           // s2 * 2^-Gs < 1
    }
    s_p[wave][lane] = __builtin_bit_cast(uint2, pw);
    if (grp == 0) s_mp[wave][row] = m_self;
    if (lane == 0) s_gp[wave] = g_self;
    pair_publish(2 * k + 1);
    // ---- this load buffer's next page
    fetch(k + kBufs, op);
    __builtin_amdgcn_sched_barrier(0);
    pair_wait(2 * k + 1);   // the partner's rows and P of the step are in place
    __builtin_amdgcn_sched_barrier(0);
    // ---- PV over the pair's two pages, this wave's half of the latent
    // (the highest priority while the multiplies issue, so the other wave of
    // the SIMD fills the matrix unit's busy cycles with its vector work)
    __builtin_amdgcn_s_setprio(2);
    v4h pother = __builtin_bit_cast(v4h, s_p[partner][lane]);
    const float m_other = s_mp[partner][row];
    const int g_other = s_gp[partner];
    constexpr int kLook = 4;   // operand reads in flight ahead of their MFMAs
    v4s va0[16], va1[16];
    auto read_tile = [&](int q) {
      va0[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(rd0 + 512 * q));
      va1[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(rd1 + 512 * q));
    };
    // the pair's common m and Gs after this step; rescales are powers of two
    const float m_new = fmaxf(m_self, m_other);
    const int g_new = max(g_self, g_other);
    // the accumulator rescale is a branch of its own, ahead of everything
    // else the rescale changes: with more work in the same branch the
    // compiler moved all 64 accumulator registers at the join on every step
    const bool resc = __ballot(m_new != m_run || g_new != Gs) != 0;
    if (resc) {
      const float f_o =
          (m_run == -INFINITY || Gs == kGUnset) ? 0.0f : pow2i(m_run + (float)Gs - (m_new + (float)g_new));
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t] *= f_o;
    }
#pragma unroll
    for (int q = 0; q < kLook; ++q) read_tile(q);
    if (resc) {
      const float e_new = m_new + (float)g_new;
      l_run = (m_run == -INFINITY ? 0.0f : l_run * pow2i(m_run - m_new)) +
              (m_self == -INFINITY ? 0.0f : psum * pow2i(m_self - m_new));
      const float f_self = (m_self == -INFINITY || g_self == kGUnset) ? 0.0f : pow2i(m_self + (float)g_self - e_new);
      const float f_other =
          (m_other == -INFINITY || g_other == kGUnset) ? 0.0f : pow2i(m_other + (float)g_other - e_new);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[i] = (_Float16)((float)pw[i] * f_self);
        pother[i] = (_Float16)((float)pother[i] * f_other);
      }
      m_run = m_new;
      Gs = g_new;
    } else {
      l_run += psum;
    }
    const v4h p0 = half == 0 ? pw : pother;
    const v4h p1 = half == 0 ? pother : pw;
    const v8h pb = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q + kLook < 16) read_tile(q + kLook);
      const v8h va = __builtin_shufflevector(__builtin_bit_cast(v4h, va0[q]), __builtin_bit_cast(v4h, va1[q]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
      o[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[q], 0, 0, 0);
      // keep the reads kLook tiles ahead instead of letting the scheduler
      // hoist all of them (64 registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    pair_publish(2 * k + 2);
  };

  // page slot k sits in load buffer k % kBufs
  int it = 0;
  for (; it + kBufs - 1 < nsteps; it += kBufs) {
#pragma unroll
    for (int j = 0; j < kBufs; ++j) step(bufs[j], it + j);
  }
#pragma unroll
  for (int j = 0; j < kBufs - 1; ++j)
    if (it + j < nsteps) step(bufs[j], it + j);

  // ---- merge the pairs. Pair totals per head: l_abs = 2^m (l_half0 +
  // l_half1), O_abs = 2^(m + Gs) O_acc.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const bool has_o = m_run != -INFINITY && Gs != kGUnset;
  const float my_e = has_o ? m_run + (float)Gs : -INFINITY;
  if (stuck) s_err = 1;
  if (grp == 0) {
    s_l[wave][row] = l_run;
    if (half == 0) {
      s_m[pair][row] = m_run;
      s_e[pair][row] = my_e;
    }
  }
  __syncthreads();   // also: every wave is past its last row read
  // a pair wait that gave up leaves NaN outputs (or NaN partials, which the
  // combine turns into NaN outputs) rather than silently wrong values
  const bool failed = s_err != 0;
  float E = -INFINITY;
#pragma unroll
  for (int q = 0; q < kPairs; ++q) E = fmaxf(E, s_e[q][row]);
  {
    const float f = my_e == -INFINITY ? 0.0f : pow2i(my_e - E);
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q] *= f;
  }
  // the per-head factors of the output pass, once per head: M and E are the
  // largest of the four pairs' m and m + Gs, den = sum over pairs of
  // 2^(m - M) (l_half0 + l_half1); with one split the output scale is
  // 2^(E - M) / den
  if (wave == 0 && lane < kHeads) {
    const int hd = lane;
    float Mh = -INFINITY, Eh = -INFINITY, den = 0.0f;
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr) {
      Mh = fmaxf(Mh, s_m[pr][hd]);
      Eh = fmaxf(Eh, s_e[pr][hd]);
    }
    if (Mh != -INFINITY) {
#pragma unroll
      for (int pr = 0; pr < kPairs; ++pr)
        if (s_m[pr][hd] != -INFINITY)
          den += __builtin_amdgcn_exp2f(s_m[pr][hd] - Mh) * (s_l[2 * pr][hd] + s_l[2 * pr + 1][hd]);
    }
    float sc = 0.0f;
    if (den > 0.0f && Eh != -INFINITY) sc = __builtin_ldexpf(1.0f / den, (int)(Eh - Mh));
    s_hf[hd] = splits == 1 ? v4f{sc, 0.0f, 0.0f, 0.0f} : v4f{Mh, den, Eh, 0.0f};
  }
  // every wave leaves its scaled half of O in LDS (tile-major, lane-minor:
  // conflict-free 16-byte writes); the output pass adds the four pairs
  v4f *slab = (v4f *)smem;   // [wave][16 tiles][64 lanes]
#pragma unroll
  for (int q = 0; q < 16; ++q) slab[(wave * 16 + q) * 64 + lane] = o[q];
  __syncthreads();
  // output: per thread and pass one slab entry (half h, tile q, lane ln:
  // dims 256h + 16q + 4(ln/16) .. +4 of head ln%16); consecutive threads read
  // consecutive entries, so the four pair reads are conflict-free
  for (int e = threadIdx.x; e < 2 * 16 * 64; e += kThreads) {
    const int h = e >> 10;
    const int q = (e >> 6) & 15;
    const int ln = e & 63;
    const int hd = ln & 15;
    const int d = kHalf * h + 16 * q + 4 * (ln >> 4);
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr) acc += slab[((2 * pr + h) * 16 + q) * 64 + ln];
    const v4f hf = s_hf[hd];
    if (splits == 1) {
      const float sc = hf[0];
      uint2 w;
      w.x = f32_to_bf16_bits(acc[0] * sc) | (f32_to_bf16_bits(acc[1] * sc) << 16);
      w.y = f32_to_bf16_bits(acc[2] * sc) | (f32_to_bf16_bits(acc[3] * sc) << 16);
      if (failed) w = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
      *(uint2 *)(a.out + ((size_t)qrow * a.hq + hd) * kLat + d) = w;
    } else {
      const size_t pi = ((size_t)b * a.hq + hd) * splits + split;
      *(v4f *)(a.part_o + pi * kLat + d) = failed ? v4f{NAN, NAN, NAN, NAN} : acc;
      if (d == 0) *(v4f *)(a.part_ml + 4 * pi) = hf;
    }
  }
}

// Split combine: per (sequence, head), out = 2^(E - M) * sum_s 2^(E_s - E) O_s
// / sum_s 2^(M_s - M) den_s, summed in split order. Splits that saw no key
// (M_s = -inf, den_s = 0) and splits with no nonzero term (E_s = -inf) drop
// out. One thread per 4 dims.
constexpr int kCombineThreads = kLat / 4;
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(const float *part_o, const float *part_ml,
                                                                      uint16_t *out, int batch, int splits) {
  int b, h;
  xcd_local(blockIdx.x, batch, kHeads, b, h);    // on the XCD that wrote sequence b's partials
  const int bh = b * kHeads + h;
  const int t = threadIdx.x;
  const float *ml = part_ml + (size_t)bh * splits * 4;
  const float *po = part_o + (size_t)bh * splits * kLat + 4 * t;
  // Every thread requests the split statistics (the same addresses for the
  // whole workgroup) and its dims' partials of the first kPre splits in one
  // memory round trip, then weighs them itself in split order: no exchange
  // between threads. Clamped copies past the last split are not used.
  constexpr int kPre = 8;
  v4f pre[kPre], st[kPre];
#pragma unroll
  for (int s = 0; s < kPre; ++s) {
    const int c = min(s, splits - 1);
    st[s] = *(const v4f *)(ml + 4 * c);
    pre[s] = *(const v4f *)(po + (size_t)c * kLat);
  }
  float M = -INFINITY, E = -INFINITY;
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < splits) {
      M = fmaxf(M, st[s][0]);
      E = fmaxf(E, st[s][2]);
    }
  for (int s = kPre; s < splits; ++s) {
    const v4f r = *(const v4f *)(ml + 4 * s);
    M = fmaxf(M, r[0]);
    E = fmaxf(E, r[2]);
  }
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
  auto add = [&](const v4f &r, const v4f &o) {
    if (r[0] != -INFINITY) den += __builtin_amdgcn_exp2f(r[0] - M) * r[1];
    if (r[2] != -INFINITY) acc += __builtin_ldexpf(1.0f, max((int)(r[2] - E), -200)) * o;
  };
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < splits) add(st[s], pre[s]);
  for (int s = kPre; s < splits; ++s) add(*(const v4f *)(ml + 4 * s), *(const v4f *)(po + (size_t)s * kLat));
  const float f = (den > 0.0f && E != -INFINITY) ? __builtin_ldexpf(1.0f / den, (int)(E - M)) : 0.0f;
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
                     a.part_o, a.part_ml, a.out, a.batch, p.splits);
  return hipGetLastError();
}

}  // namespace kvq
