// Shared device helpers and the context split policy for the paged decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kWave = 64;

// Split policy.  A sequence of ctx tokens is cut into at most `target`
// contiguous token ranges ("splits") of split_tokens tokens each (a multiple of
// kChunkTokens, so every split starts on a block boundary for block sizes 16
// and 32), and no split is shorter than kMinSplitTokens unless the whole
// context is.  Each split becomes one workgroup per KV head; the splits of a
// (sequence, KV head) are merged by log-sum-exp.  The host picks `target`:
// either from the GPU's resident-workgroup capacity and the batch's number of
// (sequence, KV head) pairs, or kMaxSplits when results must not depend on the
// rest of the batch.
constexpr int kMaxSplits = 64;        // also the final merge's lanes per head
constexpr int kMinSplitTokens = 128;
constexpr int kChunkTokens = 32;      // tokens one wave handles per iteration

struct SplitPlan {
  int num_splits;
  int split_tokens;
};

__host__ __device__ inline SplitPlan split_plan(int ctx, int target = kMaxSplits) {
  if (ctx <= 0) return {0, 0};
  int n = (ctx + kMinSplitTokens - 1) / kMinSplitTokens;
  if (n > target) n = target;
  if (n < 1) n = 1;
  int st = (ctx + n - 1) / n;
  st = (st + kChunkTokens - 1) / kChunkTokens * kChunkTokens;
  return {(ctx + st - 1) / st, st};
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 += a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Exact bf16 -> fp32 widening of the low / high half of a packed word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four OCP E4M3 codes -> four fp32 values (exact), via the gfx950 converter.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace gqa
