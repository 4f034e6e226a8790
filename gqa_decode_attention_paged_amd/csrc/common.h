// Shared device helpers and the context split policy for the paged decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kWave = 64;

// Split policy.  A sequence of ctx tokens is cut into at most `target`
// contiguous token ranges ("splits") of split_tokens tokens each (a multiple of
// kChunkTokens, so every split starts on a block boundary for block sizes 16
// and 32), and no split is shorter than `min_tokens` (kMinSplitTokens unless
// a split-length override is set) unless the whole context is.  Each split
// becomes one workgroup per KV head; the splits of a (sequence, KV head) are
// merged by log-sum-exp.  The host picks `target`: either from the GPU's
// resident-workgroup capacity and the batch's number of (sequence, KV head)
// pairs, or kMaxSplits when results must not depend on the rest of the batch.
constexpr int kMaxSplits = 64;        // also the final merge's lanes per head
constexpr int kMinSplitTokens = 128;
constexpr int kChunkTokens = 32;      // tokens one wave handles per iteration

struct SplitPlan {
  int num_splits;
  int split_tokens;
};

__host__ __device__ inline SplitPlan split_plan(int ctx, int target = kMaxSplits,
                                                int min_tokens = kMinSplitTokens) {
  if (ctx <= 0) return {0, 0};
  int n = (ctx - 1) / min_tokens + 1;              // ceil(ctx / min_tokens), no overflow
  if (n > target) n = target;
  if (n < 1) n = 1;
  int st = (ctx - 1) / n + 1;
  st = (st + kChunkTokens - 1) / kChunkTokens * kChunkTokens;
  return {(ctx - 1) / st + 1, st};
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

constexpr float kFp8Max = 448.0f;

// The smallest power of two >= t, for finite t >= 0 (0 stays 0).
__device__ __forceinline__ float pow2_ceil(float t) {
  const uint32_t u = __float_as_uint(t);
  if ((u & 0x7fffffu) == 0) return t;
  return __uint_as_float((u & 0x7f800000u) + 0x800000u);
}

// Four values -> four E4M3 codes of clamp(x / s, -448, 448) in one word (s == 0:
// zeros).  One IEEE fp32 division per value; the gfx950 converter rounds to
// nearest even.
__device__ __forceinline__ uint32_t encode4_e4m3(const float* x, float s) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = s > 0.f ? __builtin_fminf(__builtin_fmaxf(x[i] / s, -kFp8Max), kFp8Max) : 0.f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  return static_cast<uint32_t>(w);
}

// One wave appends n new bf16 rows (row j at rows + j * row_stride) to slots
// first .. first + n - 1 of one E4M3 (block, KV head) tile with its scale:
// t = max|new| / 448; a block opening here (first == 0) takes pow2_ceil(t); one
// holding older tokens keeps its scale when that is >= t, else takes
// pow2_ceil(t) and re-encodes its older codes as encode(decode(c) * old / s).
// Returns the new scale (the same in every lane).
__device__ __forceinline__ float wave_append_fp8(uint8_t* tile, float* scale_ptr, int first, int n,
                                                 const uint16_t* rows, size_t row_stride, int D,
                                                 int lane) {
  const int quads = D / 4;
  float am = 0.f;
  for (int e = lane; e < n * quads; e += kWave) {
    const uint2 w = *reinterpret_cast<const uint2*>(rows + (size_t)(e / quads) * row_stride +
                                                    (e % quads) * 4);
    am = __builtin_fmaxf(am, __builtin_fmaxf(
        __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.x)), __builtin_fabsf(bf16_hi(w.x))),
        __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.y)), __builtin_fabsf(bf16_hi(w.y)))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o));
  const float old = *scale_ptr;
  const float t = am / kFp8Max;
  const float s = (first > 0 && old >= t) ? old : pow2_ceil(t);
  uint32_t* w32 = reinterpret_cast<uint32_t*>(tile);
  if (first > 0 && t > old) {
    for (int e = lane; e < first * quads; e += kWave) {
      float v[4];
      fp8x4_to_f32(w32[e], v);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = v[i] * old;
      w32[e] = encode4_e4m3(v, s);
    }
  }
  for (int e = lane; e < n * quads; e += kWave) {
    const int j = e / quads, c = e % quads;
    const uint2 w = *reinterpret_cast<const uint2*>(rows + (size_t)j * row_stride + c * 4);
    const float v[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    w32[(size_t)(first + j) * quads + c] = encode4_e4m3(v, s);
  }
  if (lane == 0) *scale_ptr = s;
  return s;
}

// One wave appends n new rows to one (block, KV head) tile of a KIVI pool.  Keys:
// lane d' covers channels d', d' + 64, ...; each channel follows the rule of
// wave_append_fp8 on its own column (k_scale: the tile's D channel scales).
// Values: each new row gets pow2_ceil(max|row| / 448), set once (v_scale: the
// tile's BS slot scales).  Kept out of line: inlined into the decode kernel its
// loops changed the attention loop's register allocation and cost 11 us (15%)
// per step at the 40-head MHA shape even when nothing was appended.
__device__ __attribute__((noinline)) void wave_append_fp8_kivi(uint8_t* ktile, uint8_t* vtile, float* k_scale,
                                                     float* v_scale, int first, int n,
                                                     const uint16_t* krows, const uint16_t* vrows,
                                                     size_t row_stride, int D, int lane) {
  for (int d = lane; d < D; d += kWave) {
    float am = 0.f;
    for (int j = 0; j < n; ++j)
      am = __builtin_fmaxf(am, __builtin_fabsf(__uint_as_float((uint32_t)krows[j * row_stride + d] << 16)));
    const float old = k_scale[d];
    const float t = am / kFp8Max;
    const float s = (first > 0 && old >= t) ? old : pow2_ceil(t);
    if (first > 0 && t > old) {
      for (int j = 0; j < first; ++j) {
        const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(ktile[(size_t)j * D + d]), false);
        const float v[4] = {f[0] * old, 0.f, 0.f, 0.f};
        ktile[(size_t)j * D + d] = (uint8_t)(encode4_e4m3(v, s) & 0xff);
      }
    }
    for (int j = 0; j < n; ++j) {
      const float v[4] = {__uint_as_float((uint32_t)krows[j * row_stride + d] << 16), 0.f, 0.f, 0.f};
      ktile[(size_t)(first + j) * D + d] = (uint8_t)(encode4_e4m3(v, s) & 0xff);
    }
    k_scale[d] = s;
  }
  for (int j = 0; j < n; ++j) {
    float am = 0.f;
    for (int d = lane; d < D; d += kWave)
      am = __builtin_fmaxf(am, __builtin_fabsf(__uint_as_float((uint32_t)vrows[j * row_stride + d] << 16)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o));
    const float s = pow2_ceil(am / kFp8Max);
    for (int q = lane; q < D / 4; q += kWave) {
      const uint2 w = *reinterpret_cast<const uint2*>(vrows + j * row_stride + q * 4);
      const float v[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
      reinterpret_cast<uint32_t*>(vtile + (size_t)(first + j) * D)[q] = encode4_e4m3(v, s);
    }
    if (lane == 0) v_scale[first + j] = s;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace gqa
