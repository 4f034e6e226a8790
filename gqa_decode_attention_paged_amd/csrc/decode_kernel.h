// Paged GQA decode attention: one fused kernel per decode step.
//
// Workgroup (split, KV head, sequence) computes, for the G query heads sharing
// the KV head, attention over one contiguous token range of the sequence (its
// "split"), then merges with the other splits of the same (sequence, KV head):
// every workgroup publishes its partial result, and the last one to arrive
// (atomic counter) combines them by log-sum-exp.  Optionally the kernel also
// commits the step's new token into the cache (fused KV append).
//
// Method (cites):
//  * scores s_t = scale <q, k_t>, softmax over t, weighted sum of v_t; query
//    head h reads KV head h / G — *The Mathematics of Transformer Inference*
//    (hs-black) §1, §4, §5; *Module 10: Inference and Deployment Serving*
//    (wrwei.github.io), Lab 2 (each KV head repeated over consecutive heads).
//  * K/V rows come through the block table, valid tokens only — *Module 10*,
//    "Mapping logical positions to physical blocks"; *The Mathematics of
//    Transformer Inference* §9.
//  * per-chunk running max, exponential sum and unnormalised output — the
//    online-softmax update of *LLM Inference Systems Engineering*
//    (jasonzhang109) §2.8.3; splits merged by log-sum-exp as for sequence-
//    sharded KV, *The Mathematics of Transformer Inference* §8.
//  * the step commits the new token, then its query attends over the cache
//    including it — *LLM Inference Systems Engineering* §2.1.3.
//  * fp8 K/V dequantised in-kernel with a per-(block, head) scale — *The
//    Mathematics of Transformer Inference* §11.
//
// gfx950 mapping.  A (block, KV head) tile is BS contiguous rows of D elements.
// A wave walks its chunks of CT tokens with the next chunk's loads in flight
// while the current one is computed; the chunk's block ids come from one vector
// load per wave, read out with readlane, and every tile is read through a
// buffer resource whose base is wave-uniform.  Two compute paths:
//
//  * Matrix path (bf16 pools, G >= 2).  Scores of a 16-token tile are one
//    16x16x32 bf16 MFMA product per 32 dims, C[t][g] = K q^T: each lane loads
//    16 B of one K row straight into the A-operand layout, q of the G heads is
//    the B operand (columns >= G are zero).  The softmax runs in the product's
//    output layout.  V rows are staged in LDS and read back with the gfx950
//    transpose read, which hands each lane 4 consecutive tokens of one
//    dimension: the B operand of C[g][d] += P V.  The weights P (fp32) enter as
//    two bf16 operands, the rounded value and the rounded remainder, so the
//    product carries them to about 16 significant bits; K, V and q are bf16
//    already, so every product is exact and sums are fp32.
//  * Vector path (fp8 pools, and G = 1 where 15 of 16 MFMA columns would idle).
//    LPT = D/8 lanes cover one token row, 8 elements each (16 B bf16 / 8 B fp8),
//    so one load instruction reads TPI = 64/LPT whole rows.  Partial dot
//    products of each lane's 8 dims go through LDS so that every lane finishes
//    whole (token, head) scores; value sums use fp32 FMAs on the widened rows.
//
// Waves merge through LDS, splits through the workspace (see above).
//
// The running max moves lazily: only when a chunk's max exceeds the reference
// by more than 2^kLazyLog2 in weight, so weights stay <= 256; o/l and m + log2 l
// are exact for any reference, so this only skips rescales.
#pragma once

#include <type_traits>

#include "common.h"
#include "gqa_paged.h"

namespace gqa {

// Kernel arguments other than the ones a workgroup's first loads depend on.
// Those (the block tables, context lengths, the launch's length bound, the
// table row length, the window, the split target and Q) come first as scalar
// arguments: built with kernel-argument preloading, gfx950 places them in SGPRs
// when a wave launches, so the block-id prefetch (and, on the matrix path, the
// length load) does not wait for the argument segment to load.
struct DecodeParams {
  const uint16_t* q;            // [B][Q][Hq][D] bf16
  void* k_cache;                // [NB][Hkv][BS][D]; written only by the fused append
  void* v_cache;
  float* k_scale;               // [NB][Hkv] (fp8 only); written only by the fused append
  float* v_scale;
  const uint16_t* k_new;        // fused append rows: [B][Hkv][D], or [B][Q][Hkv][D] with
  const uint16_t* v_new;        //   append_tail; else null
  const int32_t* positions;     // [B] slot of the appended token, or null
  int32_t append_tail;          // 1: commit k_new/v_new row i at position ctx - Q + i
  float* out;                   // [B][Q][Hq][D]
  float* out_lse;               // [B][Q][Hq] or null
  float* ws_o;                  // [B][Hkv][max_splits][M][D] partial outputs (normalised)
  float* ws_lse;                // [B][Hkv][max_splits][M]    partial base-2 lse
  uint32_t* counters;           // [B][Hkv] arrivals, kCounterStride words apart; zero between calls
  uint32_t* status;             // sticky GQA_STATUS_* bits (a word in the first counter's line)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                // G = num_q_heads / num_kv_heads (a power of two)
  int32_t group_shift;          // log2(G)
  int32_t rows;                 // R = G * Q rows per (sequence, KV head)
  int32_t num_blocks;
  int32_t max_splits;           // row stride of the split partials
  int32_t proportional;         // slots shared out by sequence length (2 <= B <= 64)
  int32_t defer_merge;          // 1: publish the partials only; merge_splits_kernel merges
  float scale_log2;             // softmax_scale * log2(e)
};

// Word of each (sequence, KV head) counter line that holds its split count when
// the merge is deferred to merge_splits_kernel (word 0 is the arrival counter;
// the first line's word 1 is the status word).
constexpr int kSplitCountWord = 2;

constexpr float kLazyLog2 = 8.0f;
// Arrival counters sit 256 B apart: the splits of every (sequence, KV head)
// bump their counter at about the same moment, and counters sharing a cache
// line would serialise all of those atomics.
constexpr int kCounterStride = 64;
constexpr int kMergeBatch = 16;     // partial loads in flight per thread in the final merge
constexpr float kLn2 = 0.69314718055994530942f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT lanes of a token row (LPT = 8 or 16); same bits in every lane.
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);        // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);        // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);       // row_half_mirror
  if constexpr (LPT == 16) x += dpp<0x140>(x);   // row_mirror
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// Wave-wide sum in double; exact (hence order-independent) for integer values
// whose sum stays below 2^53.
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// Cross-workgroup publication of split partials without flushing L2.  Partial
// results are written and read with agent-scope coherent accesses (the sc1
// cache policy: relaxed agent-scope atomic stores/loads, and 128-bit buffer
// loads carrying the same policy), so no L2 writeback or invalidate is needed;
// the writer waits for its stores to complete before the arrival counter is
// bumped, and the reader only loads after it has seen the last arrival.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): every vector memory access of this wave (stores included) done.
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Record a bad device-resident input in the workspace's status word (a vector
// atomic OR, issued by one lane; the bits stay set until the host clears them).
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits) {
  __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCachePolicySc1 = 16;         // buffer instruction cache-policy bit "sc1"
// Cache-policy bit "nt" (non-temporal) for the K/V tile loads: every tile is
// read once per step, and with the streaming hint the large-context workloads
// read the pools 5-9% faster (the other policy bits measure the same).
constexpr int kStreamOnce = 2;
constexpr int kBufferRsrcWord3 = 0x00020000;  // raw 32-bit buffer resource (gfx9 family)

template <bool FP8>
struct KVTraits {
  using Vec = uint4;                 // 8 bf16
  static constexpr int kBytes = 2;
};
template <>
struct KVTraits<true> {
  using Vec = uint2;                 // 8 fp8 codes
  static constexpr int kBytes = 1;
};

template <bool FP8>
__device__ __forceinline__ void widen8(const typename KVTraits<FP8>::Vec& v, float* f) {
  if constexpr (FP8) {
    fp8x4_to_f32(v.x, f);
    fp8x4_to_f32(v.y, f + 4);
  } else {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
}

// Copy the appended token's K and V rows of (b, kvh) into the cache (bf16 pools).
__device__ __forceinline__ void append_rows(const DecodeParams& p, const int32_t* block_tables,
                                            int max_blocks, int b, int kvh, int pos, int D,
                                            int BS) {
  const int units = D / 8;
  if ((int)threadIdx.x >= units || pos < 0) return;
  const int blk = pos < max_blocks * BS ? block_tables[(size_t)b * max_blocks + pos / BS] : -1;
  if (blk < 0 || blk >= p.num_blocks) {            // past the table, or not a block of the pool
    if (threadIdx.x == 0) raise_status(p.status, GQA_STATUS_BAD_APPEND);
    return;
  }
  const size_t src = ((size_t)b * p.num_kv_heads + kvh) * D + threadIdx.x * 8;
  const size_t dst = (((size_t)blk * p.num_kv_heads + kvh) * BS + pos % BS) * D + threadIdx.x * 8;
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.k_cache) + dst) =
      *reinterpret_cast<const uint4*>(p.k_new + src);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.v_cache) + dst) =
      *reinterpret_cast<const uint4*>(p.v_new + src);
}

// Cross-lane reductions.  `ror<N>`: rotate within each 16-lane row (DPP);
// `swap16`/`swap32`: exchange rows 0<->1, 2<->3 / halves (gfx950 permlane swaps).
template <int N>
__device__ __forceinline__ float ror(float x) { return dpp<0x120 + N>(x); }

__device__ __forceinline__ float max_swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_swap16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_swap16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum over the lanes l' = l (mod M) of the wave (M = 1, 2, 4, 8, 16); every
// lane receives the result for its own class.
template <int M>
__device__ __forceinline__ float class_max(float x) {
  if constexpr (M <= 1) x = fmaxf(x, ror<1>(x));
  if constexpr (M <= 2) x = fmaxf(x, ror<2>(x));
  if constexpr (M <= 4) x = fmaxf(x, ror<4>(x));
  if constexpr (M <= 8) x = fmaxf(x, ror<8>(x));
  return max_swap32(max_swap16(x));
}
template <int M>
__device__ __forceinline__ float class_sum(float x) {
  if constexpr (M <= 1) x += ror<1>(x);
  if constexpr (M <= 2) x += ror<2>(x);
  if constexpr (M <= 4) x += ror<4>(x);
  if constexpr (M <= 8) x += ror<8>(x);
  return sum_swap32(sum_swap16(x));
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Eight elements as a bf16 MFMA operand: bf16 bits as they are, or eight E4M3
// codes widened exactly (an E4M3 value has at most 4 significant bits, so the
// upper half of its fp32 form is its bf16 form; v_perm packs two upper halves).
__device__ __forceinline__ bf16x8_t widen_to_bf16x8(uint4 v) { return as_bf16x8(v); }
__device__ __forceinline__ bf16x8_t widen_to_bf16x8(uint2 v) {
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = h ? v.y : v.x;
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x), false);   // codes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x), true);    // codes 2, 3
    w[2 * h] = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u);
    w[2 * h + 1] =
        __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

// gfx950 LDS transpose read of 16-bit elements.  Within each 16-lane group, lane
// 16q + 4r + c receives element c of the 8-byte pieces addressed by lanes
// 16q + 4k + r, k = 0..3.  So when those lanes address row t0 + k, column n0 + 4r
// of a row-major bf16 tile, this lane receives rows t0 .. t0+3 of column
// n0 + 4r + c: four consecutive tokens of one dimension.
__device__ __forceinline__ i16x4_t lds_read_transposed(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
}

// KV: 0 bf16 pools; 1 fp8 pools with one scale per (block, KV head); 2 fp8 pools
// with the KIVI layout (keys scaled per channel of each (block, KV head), values
// per token).
template <int D, int BS, int M, int KV, int WAVES>
// Launch bounds ask for two resident waves per SIMD (one 8-wave or two 4-wave
// workgroups per CU), which caps registers at 256 per lane; variants of more
// than 16 rows (two row tiles) need more and run one 4-wave workgroup per CU.
//
// block_tables [B][max_blocks]; context_lens [B]; hint_ctx: the host's bound on
// the context lengths (it sizes the grid); window: sliding window w (0: the
// whole context); plan_flags: the split-count target in bits 0-7, bit 8 set
// when slots are shared out by sequence length (2 <= B <= 64), and in bits
// 16-23 the number Q of query positions per sequence (its last Q tokens).
__global__ __launch_bounds__(WAVES * kWave, M > 16 ? 1 : 8 / WAVES) void paged_decode_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int32_t hint_ctx, int32_t max_blocks, int32_t window, int32_t plan_flags, DecodeParams p) {
  constexpr bool FP8 = KV != 0;
  const int target_splits = plan_flags & 0xff;
  const int Q = (plan_flags >> 16) & 0xff;   // query positions per sequence
  // Shortest split: kMinSplitTokens, or a split-length override T (T / 32 in bits
  // 9-15 and 24-31), from the preloaded word so the plan below waits for nothing.
  const int split32 = (int)((((uint32_t)plan_flags >> 9) & 0x7fu) | (((uint32_t)plan_flags >> 24) << 7));
  const int min_split_tokens = split32 ? split32 * kChunkTokens : kMinSplitTokens;
  constexpr bool KIVI = KV == 2;
  // M is the row capacity: the rows of one (sequence, KV head) are its query
  // positions times its G query heads, row m = i*G + g (R = G*Q <= M of them).
  // Two or more rows use the matrix path (bf16 pools, and fp8 pools with one
  // scale per (block, KV head)); single rows and KIVI pools the vector path.
  constexpr bool MFMA = !KIVI && M >= 2;
  // Slots shared out by sequence length.  The matrix path branches on the
  // preloaded copy of the flag (bit 8 of plan_flags), so the uniform path does
  // not wait for the argument segment; on the vector path that copy costs 16-34
  // VGPRs, enough to halve its occupancy, so it reads the one in p.
  const bool proportional = MFMA ? (plan_flags & 0x100) != 0 : p.proportional != 0;
  constexpr int LPT = D / 8;                 // lanes per token row (8 elements each)
  constexpr int TPI = kWave / LPT;           // rows per row-layout load instruction
  constexpr int CT = (MFMA || M < 8) ? 32 : 16;   // tokens per wave chunk
  constexpr int NI = CT / TPI;               // row-layout loads per chunk
  constexpr int EPC = CT >= BS ? CT / BS : 1;  // block-table entries per chunk
  constexpr int CPG = kWave / EPC;           // chunks per preloaded table group
  constexpr int ESZ = KVTraits<FP8>::kBytes;
  constexpr int NT = WAVES * kWave;
  // Vector path.  LDS score transpose: partial dot products of token t, row g,
  // lane column c at t*PSTR + g*GSTR + c; the weights p[t][g] at t*M + g.
  constexpr int NPAIR = CT * M;              // (token, row) scores per chunk
  constexpr int PPL = (NPAIR + kWave - 1) / kWave;   // scores per lane
  constexpr int TSTEP = kWave / M;           // token stride between a lane's scores
  constexpr int GSTR = LPT + 4;
  constexpr int PSTR = M * GSTR + 4;
  constexpr int kPartFloats = CT * PSTR;
  constexpr int kValuWaveBytes = (kPartFloats + NPAIR + 4 * ((M + 3) / 4)) * 4;
  // Matrix path: 16x16x32 bf16 MFMA tiles.  Staged V rows are VSTR elements
  // apart (a shift of 8 banks per row for the transpose reads).
  constexpr int KB = D / 32;                 // k-steps of the score product
  constexpr int NN = D / 16;                 // n-tiles of the value product
  constexpr int VSTR = D + 16;
  constexpr int PRS = CT + 4;                // floats per staged weight row
  constexpr int RT = MFMA ? (M + 15) / 16 : 1;   // row tiles of 16
  constexpr int WR = 16 * RT;                // weight rows staged per wave
  constexpr int kMfmaWaveBytes = CT * VSTR * 2 + WR * PRS * 4 + WR * 4;
  constexpr int kWaveBytes = MFMA ? kMfmaWaveBytes : kValuWaveBytes;
  static_assert(BS % TPI == 0 && BS % 16 == 0 && kChunkTokens % CT == 0, "tile geometry");
  static_assert(MFMA || (kWave % M == 0 && PPL * TSTEP * M >= NPAIR && M <= 16), "score mapping");
  static_assert(!MFMA || M <= 16 || M % 16 == 0, "matrix rows come in whole tiles of 16");
  static_assert(kWaveBytes % 16 == 0, "LDS alignment");
  using Vec = typename KVTraits<FP8>::Vec;

  // Workgroup -> (KV head, slot).  blockIdx.y is the KV head and the S * B
  // workgroups (x, z) of one KV head are its slots.  Uniform allocation gives
  // slot (x, z) to split x of sequence z; proportional allocation shares the
  // slots out by sequence length (below).
  const int S = gridDim.x;
  const int kvh = blockIdx.y;
  const int G = p.group;                     // query heads per KV head
  const int R = p.rows;                      // rows in use, G*Q
  const int h0 = kvh * G;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform per wave
  const int row = lane / LPT;                // row layout: token row of this lane
  const int col = lane % LPT;                // and its 8-element column

  // LDS: per-wave chunk staging during the loop; afterwards (reused) the
  // per-wave partial sums, then the split weights and float4 sums of the merge.
  constexpr int C4 = M * D / 4;                    // float4 columns of M rows
  constexpr int SP = NT >= C4 ? NT / C4 : 1;       // threads per column in the final merge
  constexpr int kAccBytes = WAVES * M * D * 4;
  constexpr int kMergeBytes = (M * kWave + 4 * ((M + 3) / 4) + 4 * SP * C4) * 4;
  constexpr int kLoopBytes = WAVES * kWaveBytes;
  constexpr int kBufA = kAccBytes > kMergeBytes ? kAccBytes : kMergeBytes;
  constexpr int kBufBytes = kBufA > kLoopBytes ? kBufA : kLoopBytes;
  __shared__ __attribute__((aligned(16))) char sm_raw[kBufBytes];
  __shared__ float sm_m[WAVES][M];
  __shared__ float sm_l[WAVES][M];
  __shared__ int sm_flag[WAVES + 1];
  float* const sm_buf = reinterpret_cast<float*>(sm_raw);
  auto sm_acc = [&](int w, int g, int d) -> float& { return sm_buf[(w * M + g) * D + d]; };
  char* const sm_wave = sm_raw + wave * kWaveBytes;   // this wave's staging area

  // Speculative block-id prefetch: most batches have every sequence at the
  // launch hint's length, where slot (x, z) is split x of sequence z under the
  // hint's split plan; the ids of this wave's chunks there are loaded together
  // with the context lengths.
  const int32_t* bt = block_tables + (size_t)blockIdx.z * max_blocks;
  auto load_ids = [&](int s0_, int s1_, int my_n_, int jbase) {
    const int jj = jbase + lane / EPC;
    const int tok = s0_ + (wave + jj * WAVES) * CT + (lane % EPC) * BS;
    return (jj < my_n_ && tok < s1_) ? bt[tok / BS] : 0;
  };
  auto wave_chunks = [&](int s0_, int s1_) {
    const int nch = (s1_ - s0_ + CT - 1) / CT;
    return wave < nch ? (nch - wave + WAVES - 1) / WAVES : 0;
  };
  // With a sliding window, a sequence's splits cover only its attended span,
  // from the start of the block holding the first token any of its queries
  // sees: blocks wholly before the window are never read.
  auto span_base = [&](int c) {
    if (window <= 0) return 0;
    const int first = c - Q + 1 - window;                  // query 0's first token
    return first > 0 ? first / BS * BS : 0;
  };
  const int hbase = span_base(hint_ctx);
  const SplitPlan hplan = split_plan(hint_ctx - hbase, target_splits, min_split_tokens);
  const int hs0 = hbase + (int)blockIdx.x * hplan.split_tokens;
  const int hs1 = min(hint_ctx, hs0 + hplan.split_tokens);
  const int hmy_n = (int)blockIdx.x < hplan.num_splits ? wave_chunks(hs0, hs1) : 0;
  int ids = load_ids(hs0, hs1, hmy_n, 0);

  // This workgroup's sequence b, its split, and the number of slots b owns.
  int b = blockIdx.z, split = blockIdx.x, slots_b = S, ctx, pos;
  // Tokens of the split read with the non-temporal hint (the rest with the
  // default policy): in a ragged batch at most the average slot's share.  The
  // hint pays while every workgroup streams, but a split longer than the
  // average reads its remainder after most workgroups have finished, and there
  // the default policy is faster: on 16 sequences of 512-8192 tokens the step
  // drops from 55.3 to 52.0 us (a paged gather by a lone workgroup measured
  // 55 GB/s with the hint against 88 without).
  int stream_tokens = INT_MAX;
  if (proportional) {
    // Lane i holds sequence i.  When the lengths differ, sequence i gets
    // n_i = 1 + floor(R c_i / sum c) slots (invalid lengths weigh 0), R the
    // largest value in [S*B - B, S*B] for which the n_i fit the S*B slots.
    // Every wave computes the same result; the sum is exact, so n_i does not
    // depend on the batch order.  Equal lengths keep the uniform plan (which
    // the sharing would also give: n_i = S).
    const int nseq = gridDim.z;
    const int ci = lane < nseq ? context_lens[lane] : 0;
    const int pi = (p.positions && lane < nseq) ? p.positions[lane] : -1;
    const int c0 = __builtin_amdgcn_readfirstlane(ci);
    if (__ballot(lane < nseq && ci != c0) != 0) {    // lengths differ: share out
      const int cw = (ci > 0 && ci <= hint_ctx && ci <= max_blocks * BS) ? ci - span_base(ci) : 0;
      const double tot = wave_sum_f64((double)cw);
      const double f = tot > 0.0 ? (double)cw / tot : 0.0;
      const int slots = S * nseq;
      stream_tokens = __builtin_amdgcn_readfirstlane((int)(tot / slots));
      int lo = slots - nseq, hi = slots;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const float cnt = lane < nseq ? (float)(1 + (int)floor((double)mid * f)) : 0.f;
        if (class_sum<1>(cnt) <= (float)slots) lo = mid; else hi = mid - 1;
      }
      const int ni = lane < nseq ? min(1 + (int)floor((double)lo * f), p.max_splits) : 0;
      int incl = ni;                                 // inclusive prefix sum over lanes
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += t;
      }
      const int slot = (int)blockIdx.x + S * (int)blockIdx.z;
      b = __builtin_amdgcn_readfirstlane(
          __builtin_popcountll(__ballot(lane < nseq && incl <= slot)));
      if (b >= nseq) return;                         // a slot the rounding left over
      split = slot - (b > 0 ? __builtin_amdgcn_readlane(incl, b - 1) : 0);
      slots_b = __builtin_amdgcn_readlane(ni, b);
      bt = block_tables + (size_t)b * max_blocks;
    }
    ctx = __builtin_amdgcn_readlane(ci, b);
    pos = __builtin_amdgcn_readlane(pi, b);
  } else {
    ctx = context_lens[b];
    pos = p.positions ? p.positions[b] : -1;
  }
  // A sequence holds its Q query positions as its last Q tokens, so 0 < ctx < Q
  // is invalid (ctx = 0 stays the empty sequence).
  const bool ctx_bad = ctx < 0 || ctx > max_blocks * BS || (ctx > 0 && ctx < Q);
  const int base = ctx_bad ? 0 : span_base(ctx);    // first token of the attended span
  const SplitPlan plan = split_plan(ctx_bad ? 0 : ctx - base,
                                    proportional ? slots_b : target_splits, min_split_tokens);
  // Whatever the plan, the last 15% of a split's tokens take the default policy
  // too: a mix of the two policies reads faster than either alone (32K step
  // 87.7 -> 85.9 us, 8K 14.15 -> 13.78 us; 0.75 and 0.9 measure slower).
  stream_tokens = min(stream_tokens, (int)(0.85f * (float)plan.split_tokens));
  // Row m of this (sequence, KV head) is query i = m / G of head h0 + m % G; its
  // flat index into q [B][Q][H_q][D], out and out_lse.  Query i sits at position
  // ctx - Q + i and attends to the tokens before it and itself.
  auto row_index = [&](int m) -> size_t {
    return ((size_t)b * Q + (m >> p.group_shift)) * p.num_q_heads + h0 + (m & (G - 1));
  };
  auto row_limit = [&](int m) { return ctx - Q + 1 + (m >> p.group_shift); };   // tokens < this
  auto row_low = [&](int m) {                      // and tokens >= this (sliding window)
    return window > 0 ? max(0, row_limit(m) - window) : 0;
  };
  const bool too_long = ctx > hint_ctx || plan.num_splits > slots_b ||
                        plan.num_splits > p.max_splits;
  const bool degenerate = ctx_bad || too_long || plan.num_splits == 0;
  const bool pos_in_split = !degenerate && pos >= base && pos < ctx;
  const int owner = pos_in_split ? (pos - base) / plan.split_tokens : 0;
  // One wave quantises new rows into one fp8 (block, KV head) tile, either layout.
  auto append_fp8_tile = [&](int blk, int first, int n, size_t row, size_t stride) {
    const size_t tile = ((size_t)blk * p.num_kv_heads + kvh) * BS * D;
    const size_t sidx = (size_t)blk * p.num_kv_heads + kvh;
    uint8_t* kt = static_cast<uint8_t*>(p.k_cache) + tile;
    uint8_t* vt = static_cast<uint8_t*>(p.v_cache) + tile;
    if constexpr (KIVI) {
      wave_append_fp8_kivi(kt, vt, p.k_scale + sidx * D, p.v_scale + sidx * BS, first, n,
                           p.k_new + row, p.v_new + row, stride, D, lane);
    } else {
      wave_append_fp8(kt, p.k_scale + sidx, first, n, p.k_new + row, stride, D, lane);
      wave_append_fp8(vt, p.v_scale + sidx, first, n, p.v_new + row, stride, D, lane);
    }
  };
  if (p.positions && split == owner && !pos_in_split) {
    if constexpr (FP8) {
      if (wave == 0 && pos >= 0) {
        const int blk = pos < max_blocks * BS ? block_tables[(size_t)b * max_blocks + pos / BS] : -1;
        if ((unsigned)blk < (unsigned)p.num_blocks)
          append_fp8_tile(blk, pos % BS, 1, ((size_t)b * p.num_kv_heads + kvh) * D, 0);
        else if (lane == 0)
          raise_status(p.status, GQA_STATUS_BAD_APPEND);
      }
    } else {
      append_rows(p, block_tables, max_blocks, b, kvh, pos, D, BS);
    }
  }

  const size_t pair_line = ((size_t)b * p.num_kv_heads + kvh) * kCounterStride;
  if (degenerate) {
    if (split != 0) return;
    if (p.defer_merge && tid == 0) p.counters[pair_line + kSplitCountWord] = 0;  // written here
    const bool bad = ctx_bad || too_long;
    if (tid == 0 && bad)
      raise_status(p.status, ctx_bad ? GQA_STATUS_BAD_CONTEXT_LEN : GQA_STATUS_CONTEXT_OVER_HINT);
    const float v = bad ? __builtin_nanf("") : 0.f;
    for (int i = tid; i < R * D; i += NT) p.out[row_index(i / D) * D + i % D] = v;
    if (p.out_lse && tid < R) p.out_lse[row_index(tid)] = bad ? __builtin_nanf("") : kNegInf;
    return;
  }
  const int nsplit = plan.num_splits;
  if (split >= nsplit) return;
  if (p.defer_merge && split == 0 && tid == 0)
    p.counters[pair_line + kSplitCountWord] = (uint32_t)nsplit;
  const int s0 = base + split * plan.split_tokens;
  const int s1 = min(ctx, s0 + plan.split_tokens);
  const int my_n = wave_chunks(s0, s1);
  int append_j = -1;                         // bf16 append: this wave's chunk holding a new row
  // Fused append: the token at `pos`, or with append_tail the Q query positions
  // ctx-Q .. ctx-1 (row i of k_new/v_new).  The wave whose chunk holds a new
  // token commits its K/V rows and waits for the stores before it issues that
  // chunk's loads, so they read the token back from the cache (bf16: append_j
  // is that chunk's index among the wave's chunks; the wait sits where its loads
  // are issued, and by then the stores have long completed: 8K step 13.33 ->
  // 13.19 us).  fp8 pools: the wave whose chunk holds a
  // block's first new token quantises that block's new rows (the append policy
  // of wave_append_fp8: its scale may grow and its older codes be re-encoded),
  // waits for the stores and invalidates the CU's vector L1, so every later
  // vector load of the tile or of its scale (buffer loads, both) reads them
  // from L2.  When a block spans several chunks (BS > CT) other waves read it
  // too, and the workgroup waits for the append before any tile is read.
  if constexpr (FP8) {
    constexpr bool kShared = BS > CT;
    const int na = p.append_tail ? Q : (pos >= 0 ? 1 : 0);
    const int a0 = p.append_tail ? ctx - Q : pos;
    const int rows_per_seq = p.append_tail ? Q : 1;
    const size_t stride = (size_t)p.num_kv_heads * D;
    bool wrote = false, any_here = false;
#pragma unroll
    for (int k = 0; k < 2; ++k) {                         // at most two blocks: Q <= BS
      const int nxt = (a0 / BS + 1) * BS;                   // start of the second block
      const int lo = k == 0 ? a0 : nxt;                    // new tokens lo .. hi-1
      const int hi = k == 0 ? min(a0 + na, nxt) : a0 + na;
      if (na <= 0 || lo >= hi || lo < s0 || lo >= s1) continue;
      const int blk = bt[lo / BS];
      if ((unsigned)blk >= (unsigned)p.num_blocks) {
        if (tid == 0) raise_status(p.status, GQA_STATUS_BAD_APPEND);
        continue;
      }
      any_here = true;
      if (((lo - s0) / CT) % WAVES != wave) continue;
      const size_t row = (((size_t)b * rows_per_seq + (lo - a0)) * p.num_kv_heads + kvh) * D;
      append_fp8_tile(blk, lo % BS, hi - lo, row, stride);
      wrote = true;
    }
    if (wrote) {
      wait_vector_memory();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");     // vector L1 invalidate
    }
    if constexpr (kShared) {
      if (any_here) __syncthreads();                       // uniform over the workgroup
    }
  } else {
    // bf16: a new row is read back only by the wave whose chunk holds it, so
    // that wave waits for its stores just before it issues that chunk's loads
    // (append_j, below), not before its first loads.
    const int na = p.append_tail ? Q : (pos >= 0 ? 1 : 0);
    const int a0 = p.append_tail ? ctx - Q : pos;
    for (int i = 0; i < na; ++i) {
      const int ap = a0 + i;
      if (ap < s0 || ap >= s1 || ((ap - s0) / CT) % WAVES != wave) continue;
      append_j = (ap - s0) / CT / WAVES;                 // this wave's chunk holding the row
      if (row != 0) continue;
      const size_t src = (((size_t)b * (p.append_tail ? Q : 1) + i) * p.num_kv_heads + kvh) * D +
                         col * 8;
      const int blk = bt[ap / BS];
      if ((unsigned)blk < (unsigned)p.num_blocks) {
        const size_t dst = (((size_t)blk * p.num_kv_heads + kvh) * BS + ap % BS) * D + col * 8;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.k_cache) + dst) =
            *reinterpret_cast<const uint4*>(p.k_new + src);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.v_cache) + dst) =
            *reinterpret_cast<const uint4*>(p.v_new + src);
      } else if (lane == 0) {
        raise_status(p.status, GQA_STATUS_BAD_APPEND);
      }
    }
  }
  if (b != (int)blockIdx.z || s0 != hs0 || s1 != hs1)
    ids = load_ids(s0, s1, my_n, 0);               // the speculation did not apply

  // Online-softmax state of the vector path (the matrix path keeps one per row
  // tile): m_ref, the reference max of this lane's head (wave-uniform per head),
  // and l_part, this lane's share of that
  // head's exponential sum.
  float m_ref = kNegInf, l_part = 0.f;
  bool bad = false;

  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  constexpr size_t kTileBytes = (size_t)BS * D * ESZ;
  const size_t block_stride = (size_t)p.num_kv_heads * kTileBytes;
  int j0 = 0;

  // Block id of table entry e of chunk j (wave-uniform, via readlane).
  auto block_id = [&](int j, int e) { return __builtin_amdgcn_readlane(ids, (j - j0) * EPC + e); };
  // One (block, KV head) tile as a buffer resource: the block id is wave-uniform,
  // so the base lives in scalar registers and each lane adds its 32-bit offset.
  auto tile_rsrc = [&](int j, int e, const char* pool, bool track) {
    int phys = block_id(j, e);
    const bool ok = (unsigned)phys < (unsigned)p.num_blocks;
    if (track) bad |= !ok;
    phys = ok ? phys : 0;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(pool) + (size_t)phys * block_stride + (size_t)kvh * kTileBytes, 0,
        (int)kTileBytes, kBufferRsrcWord3);
  };
  auto chunk_start = [&](int j) { return s0 + (wave + j * WAVES) * CT; };
  auto chunk_streams = [&](int j) { return chunk_start(j) - s0 < stream_tokens; };
  auto advance_ids = [&](int j) {        // before issuing chunk j + 1
    if (j + 1 - j0 >= CPG) {
      j0 += CPG;
      ids = load_ids(s0, s1, my_n, j0);
    }
  };
  // Row-layout loads of chunk j (V, and K on the vector path): instruction i
  // reads TPI whole rows.  Branch-free: every row reads an in-bounds slot (rows
  // past the split end read their block's unused slots, whole groups past it
  // read block 0) and compute masks them.
  const uint32_t lane_off = (uint32_t)lane * 8 * ESZ;
  // fp8 scales [NB][Hkv] as buffer resources: their loads are vector loads, which
  // after a fused append read the new scales (see above).
  // KIVI: k_scale [NB][Hkv][D], v_scale [NB][Hkv][BS].  (The host keeps these
  // byte counts below 2^31.)
  constexpr int KSPB = KIVI ? D : 1;                  // k scales per (block, KV head)
  constexpr int VSPB = KIVI ? BS : 1;                 // v scales per (block, KV head)
  const int kscale_bytes = FP8 ? p.num_blocks * p.num_kv_heads * KSPB * 4 : 0;
  const int vscale_bytes = FP8 ? p.num_blocks * p.num_kv_heads * VSPB * 4 : 0;
  const auto kscale_rsrc = __builtin_amdgcn_make_buffer_rsrc(p.k_scale, 0, kscale_bytes,
                                                             kBufferRsrcWord3);
  const auto vscale_rsrc = __builtin_amdgcn_make_buffer_rsrc(p.v_scale, 0, vscale_bytes,
                                                             kBufferRsrcWord3);
  // KIVI keys: this lane's 8 channel scales for each block of a chunk, loaded
  // with the chunk's K rows.
  constexpr int KCB = KIVI ? (CT >= BS ? CT / BS : 1) : 1;
  float kcs[KCB][8];
  // The tile loads' cache policy is an immediate, so each policy has its own
  // copy of the loads, chosen per chunk by a wave-uniform branch on the matrix
  // path.  The vector path instead runs its chunk loop in two parts, one per
  // policy: the branch costs it 14-26 VGPRs, enough to halve some variants'
  // occupancy.
  using StreamPolicy = std::integral_constant<int, kStreamOnce>;
  using DefaultPolicy = std::integral_constant<int, 0>;
  auto issue_rows_with = [&](auto policy, int j, const char* pool, Vec (&r)[NI], float (&sc)[NI],
                             bool is_k, bool track) __attribute__((always_inline)) {
    constexpr int kPolicy = decltype(policy)::value;
    const int t0 = chunk_start(j);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = CT >= BS ? (i * TPI) / BS : 0;
      const auto rsrc = tile_rsrc(j, e, pool, track);
      const int first = (t0 + i * TPI) % BS;       // first row of this instruction, uniform
      if constexpr (FP8) {
        r[i] = __builtin_bit_cast(
            Vec, __builtin_amdgcn_raw_buffer_load_b64(rsrc, lane_off, first * D * ESZ, kPolicy));
        int phys = block_id(j, e);
        phys = (unsigned)phys < (unsigned)p.num_blocks ? phys : 0;
        if constexpr (KIVI) {
          if (is_k) {
            // the block's channel scales for this lane's 8 dims, once per block
            // (per-lane part in voffset, the block's part in the uniform soffset)
            if (CT >= BS ? (i * TPI) % BS == 0 : i == 0) {
              const int tile = (phys * p.num_kv_heads + kvh) * D * 4;
              const f32x4 a = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(kscale_rsrc, col * 32, tile, 0));
              const f32x4 b = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(kscale_rsrc, col * 32 + 16, tile, 0));
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                kcs[e][k] = a[k];
                kcs[e][4 + k] = b[k];
              }
            }
          } else {
            // the value scale of this lane's token (its slot in the block)
            const int slot = (t0 + i * TPI + row) % BS;
            sc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                vscale_rsrc, slot * 4, (phys * p.num_kv_heads + kvh) * BS * 4, 0));
          }
        } else {
          sc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
              is_k ? kscale_rsrc : vscale_rsrc, 0, (phys * p.num_kv_heads + kvh) * 4, 0));
        }
      } else {
        r[i] = __builtin_bit_cast(
            Vec, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off, first * D * ESZ, kPolicy));
      }
    }
  };
  auto issue_rows = [&](int j, const char* pool, Vec (&r)[NI], float (&sc)[NI], bool is_k,
                        bool track) __attribute__((always_inline)) {
    if (!MFMA || chunk_streams(j))
      issue_rows_with(StreamPolicy{}, j, pool, r, sc, is_k, track);
    else
      issue_rows_with(DefaultPolicy{}, j, pool, r, sc, is_k, track);
  };

  bool wave_bad = false;
  if constexpr (MFMA) {
    // ---- Matrix path.  Scores C[t][g] = K q^T per 16-token tile (A = K rows,
    // B = q), value sums C[g][d] += P V (A = weights, B = V read transposed from
    // LDS).  Lane l is column hd = l & 15 and k-group qd = l >> 4 of each tile.
    // The rows come in RT tiles of 16 (rows 16 rt .. 16 rt + 15); each K and V
    // tile loaded serves all of them.
    const int hd = lane & 15;
    const int qd = lane >> 4;
    uint16_t* sm_v = reinterpret_cast<uint16_t*>(sm_wave);            // [CT][VSTR] bf16
    float* sm_pw = reinterpret_cast<float*>(sm_wave + CT * VSTR * 2);  // [WR][PRS] weights
    float* sm_alpha = sm_pw + WR * PRS;                                // [WR] rescale factors

    // K reaches the A-operand layout one of two ways.  Up to 8 rows per KV head
    // each lane loads its operand pieces straight from the pool: the product sums
    // over all D dims, so any assignment of dims to (kb, qd, element) serves if K
    // and q share it.  bf16: step kb, lane group qd holds dims 32*kb + 8*qd .. +7
    // (16-byte pieces; four lanes read 64 contiguous bytes of a row).  fp8: dims
    // 64*(kb/2) + 16*qd + 8*(kb%2) .. +7, so one 16-byte load per lane fetches two
    // steps' codes and four lanes again read 64 contiguous bytes of a row (with
    // the bf16 assignment an fp8 piece would be 8 bytes: twice the cache-line
    // requests per byte, and the 32K G = 8 fp8 step ran 62.9 against 49.5 us).
    // With 16 rows or more, K rows are loaded whole like V rows and staged through
    // LDS (STAGE_K, below), with the plain assignment.
    constexpr bool STAGE_K = M >= 16;
    constexpr bool FP8_PIECES = FP8 && !STAGE_K;
    static_assert(!FP8_PIECES || KB % 2 == 0, "fp8 K pieces hold two score steps");
    auto kdim = [&](int kb) {
      return FP8_PIECES ? 64 * (kb >> 1) + 16 * qd + 8 * (kb & 1) : 32 * kb + 8 * qd;
    };
    bf16x8_t qop[RT][KB];                 // q of row 16 rt + hd, dims kdim(kb) .. +7
    int hd_limit[RT], hd_low[RT];         // row 16 rt + hd sees tokens in [low, limit)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int m = 16 * rt + hd;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < R)
          v = *reinterpret_cast<const uint4*>(p.q + row_index(m) * D + kdim(kb));
        qop[rt][kb] = as_bf16x8(v);
      }
      hd_limit[rt] = m < R ? row_limit(m) : 0;
      hd_low[rt] = m < R ? row_low(m) : 0;
    }
    float m_t[RT], l_t[RT];               // reference max and exponential-sum share per row tile
    f32x4 acc[RT][NN];                    // rows 16 rt + 4*qd + r; columns: dims 16*n + hd
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      m_t[rt] = kNegInf;
      l_t[rt] = 0.f;
#pragma unroll
      for (int n = 0; n < NN; ++n) acc[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Direct: row (lane & 15) of a 16-token tile, dims kdim(kb) .. +7 (each
    // instruction reads 16 rows x 64 B: bf16 for one step, fp8 codes for two,
    // widened to bf16 before the product).  fp8: ks[t16] is the K scale of the
    // block holding 16-token tile t16 (a block of 16 or 32 tokens holds whole
    // tiles); it multiplies that tile's scores.
    const uint32_t k_lane_off = (uint32_t)((hd * D + (FP8_PIECES ? 16 : 8) * qd) * ESZ);
    using KOp = typename KVTraits<FP8>::Vec;  // 8 elements: uint4 (bf16) or uint2 (fp8)
    KOp kr[STAGE_K ? 1 : 2 * KB];
    float ks[FP8 ? 2 : 1];
    auto issue_k_with = [&](auto policy, int j) __attribute__((always_inline)) {
      const int t0 = chunk_start(j);
#pragma unroll
      for (int t16 = 0; t16 < 2; ++t16) {
        const int e = CT >= BS ? (16 * t16) / BS : 0;
        const auto rsrc = tile_rsrc(j, e, kbase, true);
        const int first = (t0 + 16 * t16) % BS;
        if constexpr (FP8_PIECES) {
#pragma unroll
          for (int h = 0; h < KB / 2; ++h) {       // steps 2h and 2h + 1
            const uint4 w = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, k_lane_off, first * D + 64 * h,
                                                             decltype(policy)::value));
            kr[t16 * KB + 2 * h] = make_uint2(w.x, w.y);
            kr[t16 * KB + 2 * h + 1] = make_uint2(w.z, w.w);
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            kr[t16 * KB + kb] = __builtin_bit_cast(
                KOp, __builtin_amdgcn_raw_buffer_load_b128(rsrc, k_lane_off,
                                                           (first * D + 32 * kb) * 2,
                                                           decltype(policy)::value));
        }
        if constexpr (FP8) {
          int phys = block_id(j, e);
          phys = (unsigned)phys < (unsigned)p.num_blocks ? phys : 0;
          ks[t16] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
              kscale_rsrc, 0, (phys * p.num_kv_heads + kvh) * 4, 0));
        }
      }
    };
    auto issue_k = [&](int j) __attribute__((always_inline)) {
      if constexpr (!STAGE_K) {
        if (chunk_streams(j))
          issue_k_with(StreamPolicy{}, j);
        else
          issue_k_with(DefaultPolicy{}, j);
      }
    };
    // Staged (STAGE_K): K rows are loaded like V rows (whole rows per instruction,
    // contiguous), and each chunk's rows pass through the V staging area of LDS
    // into the A-operand layout.  A paged gather in the direct pattern reads
    // 5.6-5.8 TB/s against 6.6-6.7 for whole rows; staging adds LDS latency to
    // each chunk, which pays only where the rows' compute is long anyway (16
    // rows, 8K: 18.1 -> 17.7 us; 32 rows, 32K: 93.8 -> 92.8) and costs a single
    // wave per SIMD 0.17 us per chunk at 8 rows.  fp8 codes are widened to bf16
    // on the way into LDS; ksc[i] is the K scale of row instruction i's block.
    Vec krow[STAGE_K ? NI : 1];
    float ksc[STAGE_K ? NI : 1];
    Vec vr[NI];
    float vsc[NI];                           // fp8: V scale of each row instruction's block
    uint16_t* const sm_k = sm_v;             // K rows share the staging area (K, then V, per chunk)
    const int k4 = hd >> 2, r4 = lane & 3;   // transpose-read source row / column piece

    auto run_chunk = [&](int j, auto slow_tag, auto next_tag) {
      constexpr bool SLOW = decltype(slow_tag)::value;   // split tail: rows past s1
      constexpr bool NEXT = decltype(next_tag)::value;   // chunk j+1 exists
      const int t0 = chunk_start(j);
      const int nvalid = s1 - t0;
      f32x4 sc[RT][2];
      float smul[2];                       // score multiplier of each 16-token tile
      if constexpr (STAGE_K) {
        // K rows to LDS (rows past the split end hold whatever their slots hold:
        // their scores are masked by selection below), then the next chunk's K
        // loads reuse the registers.
#pragma unroll
        for (int i = 0; i < NI; ++i)
          *reinterpret_cast<uint4*>(sm_k + (i * TPI + row) * VSTR + 8 * col) =
              __builtin_bit_cast(uint4, widen_to_bf16x8(krow[i]));
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16)
          smul[t16] = FP8 ? p.scale_log2 * ksc[t16 * (NI / 2)] : p.scale_log2;
        __builtin_amdgcn_sched_barrier(0);   // K(j+1) overwrites the rows just staged
        if constexpr (NEXT) {
          advance_ids(j);
          if (j + 1 == append_j) wait_vector_memory();   // the new row is in chunk j+1
          issue_rows(j + 1, kbase, krow, ksc, true, true);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16) {
          bf16x8_t ka[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            ka[kb] = *reinterpret_cast<const bf16x8_t*>(sm_k + (16 * t16 + hd) * VSTR +
                                                        32 * kb + 8 * qd);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            sc[rt][t16] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              sc[rt][t16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qop[rt][kb],
                                                                   sc[rt][t16], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16) {
          bf16x8_t ka[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) ka[kb] = widen_to_bf16x8(kr[t16 * KB + kb]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            sc[rt][t16] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              sc[rt][t16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qop[rt][kb],
                                                                   sc[rt][t16], 0, 0, 0);
          }
          smul[t16] = FP8 ? p.scale_log2 * ks[t16] : p.scale_log2;
        }
        __builtin_amdgcn_sched_barrier(0);   // K(j+1) overwrites the operands just used
        if constexpr (NEXT) {
          advance_ids(j);
          if (j + 1 == append_j) wait_vector_memory();   // the new row is in chunk j+1
          issue_k(j + 1);
        }
      }
      // This lane's scores: row 16 rt + hd, tokens 16*t16 + 4*qd + r.
      float s[RT][8];
      bool any_need = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int lim = min(nvalid, hd_limit[rt] - t0);  // tokens t < lim count for this row
        const int lo = hd_low[rt] - t0;                  // and t >= lo
        float cmax = kNegInf;
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * t16 + 4 * qd + r;
            float x = sc[rt][t16][r] * smul[t16];
            if (t >= lim || t < lo) x = kNegInf;  // split tail, causal limit, window, unused rows
            s[rt][t16 * 4 + r] = x;
            cmax = fmaxf(cmax, x);
          }
        cmax = max_swap32(max_swap16(cmax));   // chunk max of this row, wave-wide
        const bool need = cmax > m_t[rt] + kLazyLog2;
        if (__any(need)) {
          const float m_new = need ? cmax : m_t[rt];
          const float alpha = m_new == m_t[rt] ? 1.f : fast_exp2(m_t[rt] - m_new);
          l_t[rt] *= alpha;
          m_t[rt] = m_new;
          if (lane < 16) sm_alpha[16 * rt + lane] = alpha;
          any_need = true;
        } else if (RT > 1 && lane < 16) {
          sm_alpha[16 * rt + lane] = 1.f;
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float pw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          pw[k] = s[rt][k] > kNegInf ? fast_exp2(s[rt][k] - m_t[rt]) : 0.f;
          l_t[rt] += pw[k];
        }
        // fp8: the value sums take the weights times the V scale of the tile's
        // block (the exponential sum above takes them unscaled).  A masked token's
        // weight is 0 by selection: its tile may be a stand-in block whose scale
        // is anything, NaN included.
        if constexpr (FP8) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float vm = vsc[(k / 4) * (NI / 2)];
            pw[k] = s[rt][k] > kNegInf ? pw[k] * vm : 0.f;
          }
        }
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16)
          *reinterpret_cast<float4*>(sm_pw + (16 * rt + hd) * PRS + 16 * t16 + 4 * qd) =
              make_float4(pw[4 * t16], pw[4 * t16 + 1], pw[4 * t16 + 2], pw[4 * t16 + 3]);
      }
      // V rows to LDS (rows past the split end as zeros: their slots may hold
      // NaN poison), then the next chunk's V loads reuse the registers.
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        Vec v = vr[i];
        if (SLOW && i * TPI + row >= nvalid) v = Vec{};
        *reinterpret_cast<uint4*>(sm_v + (i * TPI + row) * VSTR + 8 * col) =
            __builtin_bit_cast(uint4, widen_to_bf16x8(v));
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NEXT) issue_rows(j + 1, vbase, vr, vsc, false, false);
      __builtin_amdgcn_wave_barrier();
      if (any_need) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float al[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) al[r] = sm_alpha[16 * rt + 4 * qd + r];
#pragma unroll
          for (int n = 0; n < NN; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rt][n][r] *= al[r];
        }
      }
      // Weights as the A operand (row 16 rt + hd, tokens 8*qd .. +7), split into a
      // bf16 high part and the bf16 rounding of the remainder: two products give
      // the weights to about 16 significant bits.
      bf16x8_t whi[RT], wlo[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float4 wa = *reinterpret_cast<const float4*>(sm_pw + (16 * rt + hd) * PRS + 8 * qd);
        const float4 wb =
            *reinterpret_cast<const float4*>(sm_pw + (16 * rt + hd) * PRS + 8 * qd + 4);
        const float wf[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          whi[rt][k] = (__bf16)wf[k];
          wlo[rt][k] = (__bf16)(wf[k] - (float)whi[rt][k]);
        }
      }
      // Value sums: the B operand (tokens 8*qd .. +7 of dim 16*n + hd) comes from
      // two transpose reads of the staged rows.
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const uint16_t* src = sm_v + (8 * qd + k4) * VSTR + 16 * n + 4 * r4;
        const i16x4_t lo = lds_read_transposed(src);
        const i16x4_t hi = lds_read_transposed(src + 4 * VSTR);
        const bf16x8_t vop =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          acc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[rt], vop, acc[rt][n], 0, 0, 0);
          acc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo[rt], vop, acc[rt][n], 0, 0, 0);
        }
      }
    };

    // Rotating pipeline: K(j+1) is issued right after the scores of chunk j,
    // V(j+1) as soon as V(j) is staged in LDS.
    if (my_n > 0) {
      if (append_j == 0) wait_vector_memory();           // the new row is in chunk 0
      if constexpr (STAGE_K)
        issue_rows(0, kbase, krow, ksc, true, true);
      else
        issue_k(0);
      issue_rows(0, vbase, vr, vsc, false, false);
    }
    for (int j = 0; j + 1 < my_n; ++j) run_chunk(j, std::false_type{}, std::true_type{});
    if (my_n > 0) {
      if (chunk_start(my_n - 1) + CT > s1)
        run_chunk(my_n - 1, std::true_type{}, std::false_type{});
      else
        run_chunk(my_n - 1, std::false_type{}, std::false_type{});
    }

    // Wave result: the products already summed over tokens; l adds over the
    // lanes of the same row.
    float l_wave[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l_wave[rt] = sum_swap32(sum_swap16(l_t[rt]));
    wave_bad = __any(bad);
    __syncthreads();                                 // staging area becomes sm_acc
    // Every row below the capacity M is stored, under one branch per row tile
    // instead of one per element: rows R..M-1 hold zeros (their weights are all
    // zero) and are never read.  Lane group qd holds rows 16 rt + 4 qd .. + 3.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (16 * rt + 4 * qd < M) {
#pragma unroll
        for (int n = 0; n < NN; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (M >= 4 || r < M) sm_acc(wave, 16 * rt + 4 * qd + r, 16 * n + hd) = acc[rt][n][r];
      }
      if (lane < 16 && 16 * rt + lane < R) {
        sm_m[wave][16 * rt + lane] = m_t[rt];
        sm_l[wave][16 * rt + lane] = l_wave[rt];
      }
    }
  } else {
    // ---- Vector path.  LPT lanes hold one token row (8 elements each); partial
    // dot products go through LDS so each lane finishes whole scores.
    float* sm_part = reinterpret_cast<float*>(sm_wave);   // transpose area
    float* sm_pw = sm_part + kPartFloats;                 // [CT][M] weights
    float* sm_alpha = sm_pw + NPAIR;                      // [M] rescale factors

    // q: this lane's 8 dims of each of the M rows (rows >= R are zero).
    uint32_t qw[M][4];
    float qf[FP8 ? M : 1][8];
#pragma unroll
    for (int g = 0; g < M; ++g) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (g < R) v = *reinterpret_cast<const uint4*>(p.q + row_index(g) * D + col * 8);
      qw[g][0] = v.x; qw[g][1] = v.y; qw[g][2] = v.z; qw[g][3] = v.w;
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qf[g][2 * j] = bf16_lo(qw[g][j]);
          qf[g][2 * j + 1] = bf16_hi(qw[g][j]);
        }
      }
    }
    // This lane's scores are for row sg = lane % M; acc holds the value sums
    // of this lane's 8 dims.
    const int sg = lane % M;
    const int sg_limit = sg < R ? row_limit(sg) : 0;     // row sg sees tokens < this
    const int sg_low = sg < R ? row_low(sg) : 0;         // and >= this
    float acc[M][8];
#pragma unroll
    for (int g = 0; g < M; ++g)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[g][k] = 0.f;
    Vec kr[NI], vr[NI];
    float ks[NI], vs[NI];

    // One chunk: partial dot products -> LDS; each lane sums and exponentiates its
    // own (token, row) scores; weights -> LDS; value sums.  SLOW handles the
    // split's tail chunk (V rows past the end are zeroed).
    auto run_chunk = [&](int j, auto slow_tag, auto next_tag, auto policy) {
      constexpr bool SLOW = decltype(slow_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;     // chunk j+1 exists
      const int t0 = chunk_start(j);
      const int nvalid = s1 - t0;                      // rows t < nvalid are real
      const int lim = min(nvalid, sg_limit - t0);      // tokens t < lim count for row sg
      const int lo = sg_low - t0;                      // and t >= lo
      if constexpr (SLOW) {
        // zero V rows past the split end (their slots may hold NaN poison)
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if (i * TPI + row >= nvalid) {
            vr[i] = Vec{};
            if constexpr (KIVI) vs[i] = 0.f;           // a slot past the end: any scale
          }
      }
      // partial dot products of this lane's 8 dims, per head
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const Vec kk = kr[i];
        float part[M];
        if constexpr (KIVI) {
          float kf[8];
          widen8<true>(kk, kf);
          const int e = CT >= BS ? (i * TPI) / BS : 0;      // constant once unrolled
#pragma unroll
          for (int k = 0; k < 8; ++k) kf[k] *= kcs[e][k];
#pragma unroll
          for (int g = 0; g < M; ++g) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) a = fmaf(qf[g][k], kf[k], a);
            part[g] = a;
          }
        } else if constexpr (FP8) {
          float kf[8];
          widen8<true>(kk, kf);
#pragma unroll
          for (int g = 0; g < M; ++g) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) a = fmaf(qf[g][k], kf[k], a);
            part[g] = a * ks[i];
          }
        } else {
#pragma unroll
          for (int g = 0; g < M; ++g) {
            float a = dot2_bf16(qw[g][0], kk.x, 0.f);
            a = dot2_bf16(qw[g][1], kk.y, a);
            a = dot2_bf16(qw[g][2], kk.z, a);
            part[g] = dot2_bf16(qw[g][3], kk.w, a);
          }
        }
        float* dst = sm_part + (i * TPI + row) * PSTR + col;
#pragma unroll
        for (int g = 0; g < M; ++g) dst[g * GSTR] = part[g];
      }
      __builtin_amdgcn_sched_barrier(0);   // keep K(j+1) behind the scores of chunk j
      if constexpr (NEXT) {
        advance_ids(j);
        if (j + 1 == append_j) wait_vector_memory();     // the new row is in chunk j+1
        issue_rows_with(policy, j + 1, kbase, kr, ks, true, true);
      }
      __builtin_amdgcn_wave_barrier();
      // this lane's scores: token t = lane / M + q * TSTEP, row sg
      float sc[PPL];
      float cmax = kNegInf;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const int t = lane / M + q * TSTEP;
        float tot = kNegInf;
        if (t < CT) {
          const float4* src = reinterpret_cast<const float4*>(sm_part + t * PSTR + sg * GSTR);
          float a = 0.f;
#pragma unroll
          for (int c4 = 0; c4 < LPT / 4; ++c4) {
            const float4 v = src[c4];
            a += (v.x + v.y) + (v.z + v.w);
          }
          tot = a * p.scale_log2;
          if (t >= lim || t < lo) tot = kNegInf;  // tail, causal limit, window, unused rows
        }
        sc[q] = tot;
        cmax = fmaxf(cmax, tot);
      }
      cmax = class_max<M>(cmax);                     // chunk max of row sg, wave-wide
      // lazy rescale: only when the chunk max passes the reference by 2^kLazyLog2
      const bool need = cmax > m_ref + kLazyLog2;
      const bool any_need = __any(need);
      if (any_need) {
        const float m_new = need ? cmax : m_ref;
        const float alpha = m_new == m_ref ? 1.f : fast_exp2(m_ref - m_new);  // 0 from -inf
        l_part *= alpha;
        m_ref = m_new;
        if (lane < M) sm_alpha[lane] = alpha;
      }
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const int t = lane / M + q * TSTEP;
        const float pw = sc[q] > kNegInf ? fast_exp2(sc[q] - m_ref) : 0.f;
        l_part += (t < CT) ? pw : 0.f;
        if (t < CT) sm_pw[t * M + sg] = pw;
      }
      __builtin_amdgcn_wave_barrier();
      if (any_need) {
        float al[M];
#pragma unroll
        for (int g = 0; g < M; ++g) al[g] = sm_alpha[g];
#pragma unroll
        for (int g = 0; g < M; ++g)
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[g][k] *= al[g];
      }
      // value sums
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[8];
        widen8<FP8>(vr[i], vf);
        float pw[M];
        const float* src = sm_pw + (i * TPI + row) * M;
        if constexpr (M % 4 == 0) {
#pragma unroll
          for (int g4 = 0; g4 < M / 4; ++g4) {
            const float4 v = reinterpret_cast<const float4*>(src)[g4];
            pw[4 * g4] = v.x; pw[4 * g4 + 1] = v.y; pw[4 * g4 + 2] = v.z; pw[4 * g4 + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int g = 0; g < M; ++g) pw[g] = src[g];
        }
#pragma unroll
        for (int g = 0; g < M; ++g) {
          // fp8: a masked token (weight 0) may sit in a stand-in block whose scale is
          // anything, NaN included, so it contributes 0 by selection.
          const float pg = FP8 ? (pw[g] != 0.f ? pw[g] * vs[i] : 0.f) : pw[g];
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[g][k] = fmaf(pg, vf[k], acc[g][k]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep V(j+1) behind the value sums of chunk j
      if constexpr (NEXT) issue_rows_with(policy, j + 1, vbase, vr, vs, false, false);
    };

    // Rotating pipeline: K(j+1) is issued right after the partial scores of chunk
    // j, V(j+1) right after its value sums, so the next chunk's loads fly during
    // compute with no extra registers.
    if (my_n > 0) {
      if (append_j == 0) wait_vector_memory();           // the new row is in chunk 0
      issue_rows(0, kbase, kr, ks, true, true);
      issue_rows(0, vbase, vr, vs, false, false);
    }
    // Only a wave's last chunk can be partial, so the loop runs the fast path
    // only, and the last chunk is peeled, which also lets every loop iteration
    // issue the next loads unconditionally (K/V registers are reused in place).
    // The cache policy is an immediate of the load instructions, so the chunks
    // whose successor streams with the hint and the rest run in two loops, one
    // copy of the loads each (a per-chunk branch cost this path 14-26 VGPRs).
    int j = 0;
    for (; j + 1 < my_n && chunk_streams(j + 1); ++j)
      run_chunk(j, std::false_type{}, std::true_type{}, StreamPolicy{});
    for (; j + 1 < my_n; ++j) run_chunk(j, std::false_type{}, std::true_type{}, DefaultPolicy{});
    if (my_n > 0) {
      if (chunk_start(my_n - 1) + CT > s1)
        run_chunk(my_n - 1, std::true_type{}, std::false_type{}, StreamPolicy{});
      else
        run_chunk(my_n - 1, std::false_type{}, std::false_type{}, StreamPolicy{});
    }

    // Wave result: rows share m_ref, so value sums add without rescaling; l adds
    // over the lanes holding the same head.
#pragma unroll
    for (int g = 0; g < M; ++g)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float x = acc[g][k];
        if constexpr (LPT == 8) x += ror<8>(x);
        x = sum_swap16(x);
        acc[g][k] = sum_swap32(x);
      }
    const float l_wave = class_sum<M>(l_part);      // lanes l = g (mod M) hold row g
    wave_bad = __any(bad);
    __syncthreads();                                 // transpose area becomes sm_acc
    if (row == 0) {
#pragma unroll
      for (int g = 0; g < M; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) sm_acc(wave, g, col * 8 + k) = acc[g][k];
    }
    if (lane < R) {
      sm_m[wave][lane] = m_ref;
      sm_l[wave][lane] = l_wave;
    }
  }
  if (lane == 0) sm_flag[wave] = wave_bad ? 1 : 0;
  __syncthreads();

  // Merge the waves: this split's normalised output and base-2 lse.
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) any_bad |= sm_flag[w];
  if (any_bad && tid == 0) raise_status(p.status, GQA_STATUS_BAD_BLOCK_ID);
  const size_t prow = ((size_t)b * p.num_kv_heads + kvh) * p.max_splits;   // partial rows
  if constexpr (M * D >= 4 * NT) {
    // Four or more elements per thread: four consecutive dims at a time, and
    // the partial goes out as 16-byte stores with the same coherent policy.
    const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
        p.ws_o + (prow + split) * M * D, 0, M * D * 4, kBufferRsrcWord3);
    for (int i4 = tid; i4 < R * D / 4; i4 += NT) {
      const int g = (i4 * 4) / D;                  // row
      const int d = (i4 * 4) % D;
      float mx = kNegInf;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) mx = fmaxf(mx, sm_m[w][g]);
      float L = 0.f;
      f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float mw = sm_m[w][g];
        const float a = mw > kNegInf ? fast_exp2(mw - mx) : 0.f;
        L = fmaf(a, sm_l[w][g], L);
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sm_acc(w, g, d));
        O.x = fmaf(a, v.x, O.x); O.y = fmaf(a, v.y, O.y);
        O.z = fmaf(a, v.z, O.z); O.w = fmaf(a, v.w, O.w);
      }
      // A row may see none of this split's tokens (a query position before the
      // split's start): its weight in the final merge is 2^-inf = 0, and its
      // partial is 0 rather than 0/0, which would poison that merge.
      // Scaling by 1/L, or by 0 (O is then 0: every weight of the row is 0), keeps
      // the LDS reads of the waves' sums out of a branch behind the weights, and
      // takes one divide instead of four.
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const f32x4 o = O * inv;
      const float lse2 = any_bad ? __builtin_nanf("") : mx + log2f(L);
      if (nsplit == 1) {
        const float nan = __builtin_nanf("");
        *reinterpret_cast<f32x4*>(p.out + row_index(g) * D + d) =
            any_bad ? f32x4{nan, nan, nan, nan} : o;
        if (p.out_lse && d == 0) p.out_lse[row_index(g)] = lse2 * kLn2;
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), dst,
                                               (g * D + d) * 4, 0, kCachePolicySc1);
        if (d == 0) store_coherent(&p.ws_lse[(prow + split) * M + g], lse2);
      }
    }
  } else {
  for (int idx = tid; idx < R * D; idx += NT) {
    const int g = idx / D;                         // row
    const int d = idx % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) mx = fmaxf(mx, sm_m[w][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float mw = sm_m[w][g];
      const float a = mw > kNegInf ? fast_exp2(mw - mx) : 0.f;
      L = fmaf(a, sm_l[w][g], L);
      O = fmaf(a, sm_acc(w, g, d), O);
    }
    const float o = O * (L > 0.f ? 1.f / L : 0.f);  // a row with no token here: 0, not 0/0
    const float lse2 = any_bad ? __builtin_nanf("") : mx + log2f(L);
    if (nsplit == 1) {
      p.out[row_index(g) * D + d] = any_bad ? __builtin_nanf("") : o;
      if (p.out_lse && d == 0) p.out_lse[row_index(g)] = lse2 * kLn2;
    } else {
      store_coherent(&p.ws_o[((prow + split) * M + g) * D + d], o);
      if (d == 0) store_coherent(&p.ws_lse[(prow + split) * M + g], lse2);
    }
  }
  }
  if (nsplit == 1) return;
  if (p.defer_merge) return;                     // merge_splits_kernel merges after this launch

  // Publish, count arrivals; the last workgroup of this (sequence, KV head) merges.
  wait_vector_memory();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&p.counters[((size_t)b * p.num_kv_heads + kvh) * kCounterStride],
                                                 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm_flag[WAVES] = prev == (uint32_t)(nsplit - 1);
  }
  __syncthreads();
  if (!sm_flag[WAVES]) return;

  // Final merge.  The partial outputs do not depend on the split weights, so
  // the first batch of them is loaded before the weights are computed, and the
  // weights' lse loads fly at the same time: one memory round trip.  Partial
  // rows are M apart; rows R..M-1 (padding when R is not a power of two) are
  // combined like the others but never stored.
  const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_o + prow * M * D, 0, nsplit * M * D * 4, kBufferRsrcWord3);
  auto store_out = [&](int c, const float4& o) {   // column c: row (4c)/D, dims 4(c % (D/4))..
    const int m = (c * 4) / D;
    if (m < R) *reinterpret_cast<float4*>(p.out + row_index(m) * D + (c * 4) % D) = o;
  };
  const int part = NT >= C4 ? tid / C4 : 0;        // this thread's splits: part, part + SP, ...
  const int c0 = NT >= C4 ? tid % C4 : tid;        // first float4 column of this thread
  // loads in flight per thread: enough for all splits when a column has many
  // threads, else kMergeBatch per round
  constexpr int MB = (kMaxSplits + SP - 1) / SP < kMergeBatch ? (kMaxSplits + SP - 1) / SP
                                                                : kMergeBatch;
  // Only splits that exist are loaded: each load is a coherent read from memory
  // through this one compute unit, and MB covers the largest split count.
  auto load_batch = [&](int c, int sb, f32x4 (&v)[MB]) {
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int si = sb + u * SP;
      v[u] = si < nsplit ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               src, (si * C4 + c) * 16, 0, kCachePolicySc1))
                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  f32x4 v[MB];
  if (c0 < C4) load_batch(c0, part, v);

  // Split weights per row: w_s = 2^(lse_s - max) / sum, one wave per row.
  float* sm_w = sm_buf;                            // [M][64]
  float* sm_lse = sm_buf + M * kWave;              // [M] merged base-2 lse
  float4* sm_red = reinterpret_cast<float4*>(sm_buf + M * kWave + 4 * ((M + 3) / 4));
  constexpr int RPW = (M + WAVES - 1) / WAVES;    // rows per wave
  float xs[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {                  // all of this wave's lse loads at once
    const int g = wave + r * WAVES;
    xs[r] = (g < M && lane < nsplit) ? load_coherent(&p.ws_lse[(prow + lane) * M + g]) : kNegInf;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int g = wave + r * WAVES;
    if (g >= M) break;
    const float x = xs[r];
    const bool nan = __any(x != x);
    const float mx = class_max<1>(x);
    const float w = lane < nsplit ? fast_exp2(x - mx) : 0.f;
    const float L = class_sum<1>(w);
    sm_w[g * kWave + lane] = nan ? __builtin_nanf("") : w / L;
    if (lane == 0) sm_lse[g] = nan ? __builtin_nanf("") : mx + log2f(L);
  }
  __syncthreads();

  // out[g][d] = sum_s w_s o_s[g][d] over float4 columns; SP threads share a
  // column and combine through LDS.
  for (int c = c0; c < C4; c += NT >= C4 ? C4 : NT) {
    const int g = (c * 4) / D;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sb = part;;) {
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const int si = sb + u * SP;
        const float w = si < nsplit ? sm_w[g * kWave + si] : 0.f;
        o.x = fmaf(w, v[u].x, o.x);
        o.y = fmaf(w, v[u].y, o.y);
        o.z = fmaf(w, v[u].z, o.z);
        o.w = fmaf(w, v[u].w, o.w);
      }
      sb += MB * SP;
      if (sb >= nsplit) break;
      load_batch(c, sb, v);
    }
    if constexpr (SP > 1) sm_red[part * C4 + c] = o;
    else store_out(c, o);
    if (c + (NT >= C4 ? C4 : NT) < C4) load_batch(c + (NT >= C4 ? C4 : NT), part, v);
  }
  if constexpr (SP > 1) {
    __syncthreads();
    for (int c = tid; c < C4; c += NT) {
      float4 o = sm_red[c];
#pragma unroll
      for (int q = 1; q < SP; ++q) {
        const float4 v = sm_red[q * C4 + c];
        o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
      }
      store_out(c, o);
    }
  }
  if (p.out_lse && tid < R) p.out_lse[row_index(tid)] = sm_lse[tid] * kLn2;
  if (tid == 0)
    __hip_atomic_store(&p.counters[((size_t)b * p.num_kv_heads + kvh) * kCounterStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Deferred final merge (the decode launch ran with defer_merge): one wave per
// (row, KV head, sequence), spread over the GPU instead of one workgroup per
// (sequence, KV head).  The split count comes from the decode launch
// (kSplitCountWord); with fewer than two splits that launch wrote the outputs
// itself.  The weights are the log-sum-exp merge of the splits' base-2 lse; lane
// s loads split s's lse, and the float4 columns of the row are shared out over
// LG lane groups, each taking every LG-th split, so all loads fly together.
// They are issued with the split count's own load, for the splits below
// split_cap (the launch's splits per sequence, the most any sequence has unless
// the slots were shared out by length), so one memory round trip brings them
// all; slots at or past the count hold stale values, which are masked out.
// Merges splits in the order s = 0, 1, ... within a lane group, then adds the
// groups' sums.
template <int D>
__global__ __launch_bounds__(kWave) void merge_splits_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const uint32_t* __restrict__ counters, int32_t num_kv_heads, int32_t M, int32_t max_splits,
    int32_t split_cap, int32_t Q, int32_t num_q_heads, int32_t G, int32_t group_shift,
    float* __restrict__ out, float* __restrict__ out_lse) {
  constexpr int C4 = D / 4;                        // float4 columns of a row
  constexpr int LG = kWave / C4;                   // lane groups
  constexpr int PER = kMaxSplits / LG;             // splits per lane group, at most
  const int g = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const size_t pair = (size_t)b * num_kv_heads + kvh;
  const size_t prow = pair * max_splits;
  const int col = lane % C4, grp = lane / C4;
  const int nsplit = (int)counters[pair * kCounterStride + kSplitCountWord];
  const int cap = split_cap < max_splits ? split_cap : max_splits;
  float x = lane < cap ? ws_lse[(prow + lane) * M + g] : kNegInf;
  f32x4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int si = grp + u * LG;
    v[u] = si < cap ? *reinterpret_cast<const f32x4*>(ws_o + ((prow + si) * M + g) * D + 4 * col)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (nsplit < 2) return;
  if (nsplit > cap) {                              // slots shared out by length: the rest
    if (lane >= cap && lane < nsplit) x = ws_lse[(prow + lane) * M + g];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int si = grp + u * LG;
      if (si >= cap && si < nsplit)
        v[u] = *reinterpret_cast<const f32x4*>(ws_o + ((prow + si) * M + g) * D + 4 * col);
    }
  }
  if (lane >= nsplit) x = kNegInf;
  const bool nan = __any(x != x);
  float mx = x;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
  const float w = lane < nsplit ? fast_exp2(x - mx) : 0.f;
  float L = w;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) L += __shfl_xor(L, m, kWave);
  const float wn = w / L;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int si = grp + u * LG;
    const float ws = __shfl(wn, si < kWave ? si : 0, kWave);
    if (si < nsplit) {
      o.x = fmaf(ws, v[u].x, o.x); o.y = fmaf(ws, v[u].y, o.y);
      o.z = fmaf(ws, v[u].z, o.z); o.w = fmaf(ws, v[u].w, o.w);
    }
  }
#pragma unroll
  for (int m = C4; m < kWave; m <<= 1) {
    o.x += __shfl_xor(o.x, m, kWave); o.y += __shfl_xor(o.y, m, kWave);
    o.z += __shfl_xor(o.z, m, kWave); o.w += __shfl_xor(o.w, m, kWave);
  }
  // row g is query g / G of head kvh * G + g % G
  const size_t row = ((size_t)b * Q + (g >> group_shift)) * num_q_heads + kvh * G + (g & (G - 1));
  if (grp == 0) {
    const float nanf = __builtin_nanf("");
    *reinterpret_cast<f32x4*>(out + row * D + 4 * col) = nan ? f32x4{nanf, nanf, nanf, nanf} : o;
  }
  if (out_lse && lane == 0) out_lse[row] = nan ? __builtin_nanf("") : (mx + log2f(L)) * kLn2;
}

// Zero the arrival counters of a workspace (used once, before its first call).
__global__ void zero_words_kernel(uint32_t* w, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    w[i] = 0u;
}

}  // namespace gqa
