// KV append (commit new tokens of each sequence), the copy-on-write block copy,
// and a block-table gather.
//
// Cites: *LLM Inference Systems Engineering* (jasonzhang109) §2.1.3 — a decode
// step first writes the pending token's K/V into the cache, then attends;
// *The Mathematics of Transformer Inference* (hs-black) §1 — decode appends the
// new token's own K and V; *Module 10: Inference and Deployment Serving*
// (wrwei.github.io), "Mapping logical positions to physical blocks" — token t
// lives in physical block table[t / BS] at slot t % BS.
//
// Copy-on-write: *Module 10*, "Share only state with the same identity" — a
// sequence about to write into a shared block that is not yet full first gets a
// private copy; *The Mathematics of Transformer Inference* §9 (reference counts
// and copy-on-write).
//
// The bf16 append, the copy and the gather are plain byte copies in 16-byte
// units (bit-exact).  The fp8 append quantises: *The Mathematics of Transformer
// Inference* §11 (x ~ s * round(x / s), KV scales per head and per token,
// dequantisation fused into attention); the E4M3 code and its largest value
// 448 as in *Module 10*'s number-format table.
#pragma once

#include "common.h"

namespace gqa {

struct AppendParams {
  const uint16_t* k_new;        // [B][T][Hkv][D]
  const uint16_t* v_new;
  uint16_t* k_cache;            // [NB][Hkv][BS][D]
  uint16_t* v_cache;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* positions;     // [B][T]; a position outside [0, max_blocks*BS) is skipped
  int32_t num_tokens;           // T
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks;
};

// grid: (B, T) workgroups, one per new token; each thread copies 16 B units of
// the token's K and V rows.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int b = blockIdx.x;
  const size_t tok = (size_t)b * p.num_tokens + blockIdx.y;   // row of k_new / positions
  const int pos = p.positions[tok];
  if (pos < 0 || pos >= p.max_blocks * p.block_size) return;
  const int blk = p.block_tables[(size_t)b * p.max_blocks + pos / p.block_size];
  if (blk < 0 || blk >= p.num_blocks) return;
  const int slot = pos % p.block_size;
  const int upr = p.head_dim / 8;                    // 16 B units per row
  for (int u = threadIdx.x; u < p.num_kv_heads * upr; u += blockDim.x) {
    const int h = u / upr;
    const int c = u % upr;
    const size_t src = (tok * p.num_kv_heads + h) * p.head_dim + c * 8;
    const size_t dst = (((size_t)blk * p.num_kv_heads + h) * p.block_size + slot) * p.head_dim + c * 8;
    *reinterpret_cast<uint4*>(p.k_cache + dst) = *reinterpret_cast<const uint4*>(p.k_new + src);
    *reinterpret_cast<uint4*>(p.v_cache + dst) = *reinterpret_cast<const uint4*>(p.v_new + src);
  }
}

struct AppendFp8Params {
  const uint16_t* k_new;        // [B][T][Hkv][D] bf16
  const uint16_t* v_new;
  uint8_t* k_cache;             // [NB][Hkv][BS][D] E4M3 codes
  uint8_t* v_cache;
  float* k_scale;               // [NB][Hkv]
  float* v_scale;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* start;         // [B]: positions start[b] .. start[b] + T - 1; < 0: none
  int32_t num_tokens;           // T
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks;
};

__device__ __forceinline__ float workgroup_max256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// grid: (B, Hkv, 2), 256 threads; z = 0 writes K, z = 1 writes V.  The workgroup
// walks the blocks its sequence's T new tokens fall in.  Per (block, head) tile,
// with `first` the lowest slot written and t = amax(new rows) / 448:
//   first == 0 (the block opens):   s = pow2_ceil(t)
//   first > 0, old scale >= t:      s = old (older codes untouched)
//   first > 0, old scale <  t:      s = pow2_ceil(t); older codes re-encoded as
//                                   encode(decode(c) * old / s)
// then the new rows are encode(x / s) and the tile's scale becomes s.  Scales
// are powers of two, so a re-encode only shifts exponents (exact while values
// stay normal E4M3).
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(AppendFp8Params p) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const uint16_t* xnew = is_v ? p.v_new : p.k_new;
  uint8_t* pool = is_v ? p.v_cache : p.k_cache;
  float* scales = is_v ? p.v_scale : p.k_scale;
  const int st = p.start[b];
  if (st < 0) return;
  const int BS = p.block_size, D = p.head_dim, quads = D / 4;
  const int64_t end = (int64_t)st + p.num_tokens;
  const size_t row_stride = (size_t)p.num_kv_heads * D;         // between tokens of k_new
  for (int64_t pos = st; pos < end;) {
    const int64_t bi = pos / BS;
    const int first = (int)(pos % BS);
    const int n = (int)(end - pos < BS - first ? end - pos : BS - first);
    if (bi >= p.max_blocks) break;
    const int blk = p.block_tables[(size_t)b * p.max_blocks + bi];
    if ((unsigned)blk < (unsigned)p.num_blocks) {
      const uint16_t* rows = xnew + (((size_t)b * p.num_tokens + (size_t)(pos - st)) *
                                     p.num_kv_heads + h) * D;
      float* sp = scales + (size_t)blk * p.num_kv_heads + h;
      const float old = *sp;
      float am = 0.f;
      for (int e = threadIdx.x; e < n * quads; e += 256) {
        const uint2 w = *reinterpret_cast<const uint2*>(rows + (size_t)(e / quads) * row_stride +
                                                        (e % quads) * 4);
        am = __builtin_fmaxf(am, __builtin_fmaxf(
            __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.x)), __builtin_fabsf(bf16_hi(w.x))),
            __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.y)), __builtin_fabsf(bf16_hi(w.y)))));
      }
      am = workgroup_max256(am, red);            // also orders every read of *sp before its write
      const float t = am / kFp8Max;
      const bool older = first > 0;
      const float s = (older && old >= t) ? old : pow2_ceil(t);
      uint32_t* tile = reinterpret_cast<uint32_t*>(pool + ((size_t)blk * p.num_kv_heads + h) *
                                                   BS * D);
      if (older && t > old) {
        for (int e = threadIdx.x; e < first * quads; e += 256) {
          float v[4];
          fp8x4_to_f32(tile[e], v);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = v[i] * old;
          tile[e] = encode4_e4m3(v, s);
        }
      }
      for (int e = threadIdx.x; e < n * quads; e += 256) {
        const int j = e / quads, c = e % quads;
        const uint2 w = *reinterpret_cast<const uint2*>(rows + (size_t)j * row_stride + c * 4);
        const float v[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
        tile[(size_t)(first + j) * quads + c] = encode4_e4m3(v, s);
      }
      if (threadIdx.x == 0) *sp = s;
    }
    pos += n;
  }
}

// KIVI layout (k_scale [NB][Hkv][D], v_scale [NB][Hkv][BS]).  grid (B, Hkv, 2),
// 256 threads.  Keys (z = 0): thread d owns channel d of each tile its new rows
// fall in and applies the rule of kv_append_fp8_kernel to that column (t = its
// amax / 448, growth and re-encoding per channel).  Values (z = 1): each wave
// takes whole new rows; a row's scale is pow2_ceil(amax(row) / 448), set once.
__global__ __launch_bounds__(256) void kv_append_fp8_kivi_kernel(AppendFp8Params p) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int st = p.start[b];
  if (st < 0) return;
  const int BS = p.block_size, D = p.head_dim;
  const int64_t end = (int64_t)st + p.num_tokens;
  const size_t row_stride = (size_t)p.num_kv_heads * D;        // between tokens of k_new
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t pos = st; pos < end;) {
    const int64_t bi = pos / BS;
    const int first = (int)(pos % BS);
    const int n = (int)(end - pos < BS - first ? end - pos : BS - first);
    if (bi >= p.max_blocks) break;
    const int blk = p.block_tables[(size_t)b * p.max_blocks + bi];
    if ((unsigned)blk < (unsigned)p.num_blocks) {
      const size_t tile_off = ((size_t)blk * p.num_kv_heads + h) * BS * D;
      const size_t row0 = (((size_t)b * p.num_tokens + (size_t)(pos - st)) * p.num_kv_heads + h) * D;
      if (!is_v) {
        uint8_t* tile = p.k_cache + tile_off;
        const uint16_t* rows = p.k_new + row0;
        for (int d = threadIdx.x; d < D; d += 256) {
          float am = 0.f;
          for (int j = 0; j < n; ++j)
            am = __builtin_fmaxf(am, __builtin_fabsf(__uint_as_float((uint32_t)rows[j * row_stride + d] << 16)));
          float* sp = p.k_scale + ((size_t)blk * p.num_kv_heads + h) * D + d;
          const float old = *sp;
          const float t = am / kFp8Max;
          const float s = (first > 0 && old >= t) ? old : pow2_ceil(t);
          if (first > 0 && t > old) {
            for (int j = 0; j < first; ++j) {
              const uint8_t c = tile[(size_t)j * D + d];
              const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c), false);
              const float v[4] = {f[0] * old, 0.f, 0.f, 0.f};
              tile[(size_t)j * D + d] = (uint8_t)(encode4_e4m3(v, s) & 0xff);
            }
          }
          for (int j = 0; j < n; ++j) {
            const float v[4] = {__uint_as_float((uint32_t)rows[j * row_stride + d] << 16), 0.f, 0.f, 0.f};
            tile[(size_t)(first + j) * D + d] = (uint8_t)(encode4_e4m3(v, s) & 0xff);
          }
          *sp = s;
        }
      } else {
        uint8_t* tile = p.v_cache + tile_off;
        const uint16_t* rows = p.v_new + row0;
        for (int j = wave; j < n; j += 4) {                  // one wave per new row
          float am = 0.f;
          for (int d = lane; d < D; d += 64)
            am = __builtin_fmaxf(am, __builtin_fabsf(__uint_as_float((uint32_t)rows[j * row_stride + d] << 16)));
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o));
          const float s = pow2_ceil(am / kFp8Max);
          for (int q = lane; q < D / 4; q += 64) {
            const uint2 w = *reinterpret_cast<const uint2*>(rows + j * row_stride + q * 4);
            const float v[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
            reinterpret_cast<uint32_t*>(tile + (size_t)(first + j) * D)[q] = encode4_e4m3(v, s);
          }
          if (lane == 0) p.v_scale[((size_t)blk * p.num_kv_heads + h) * BS + first + j] = s;
        }
      }
    }
    pos += n;
  }
}

constexpr int kCopyThreads = 256;
constexpr int kCopySliceBytes = kCopyThreads * 16;       // 4 KiB of each pool per workgroup
constexpr int kXcds = 8;                                 // MI355X: 8 XCDs, one L2 each

struct CopyBlocksParams {
  char* k_cache;                // [NB][Hkv][BS][row_bytes]: one block is contiguous
  char* v_cache;
  float* k_scale;               // [NB][Hkv] fp8 scales, or null
  float* v_scale;
  const int32_t* src;           // [num_pairs] source block ids
  const int32_t* dst;           // [num_pairs] destination block ids
  int32_t num_blocks;
  int32_t k_scales;             // fp8 scales per block: Hkv (per (block, head)), Hkv * D (KIVI keys)
  int32_t v_scales;             //   Hkv, or Hkv * BS (KIVI values)
  int32_t slices;               // ceil(block_bytes / kCopySliceBytes)
  uint32_t work_items;          // num_pairs * slices = the grid size
  int64_t block_bytes;          // Hkv * BS * row_bytes, a multiple of 16
};

// grid: work_items workgroups in one dimension.  Work item w = pair * slices +
// slice copies byte slice `slice` of block src[pair] onto block dst[pair] in both
// pools, 16 bytes per thread, and slice 0 also copies the blocks' fp8 scales.
// Pairs with an id outside the pool, or src == dst, copy nothing.
//
// A fork lists one source for several copies, next to each other.  The
// dispatcher deals workgroups round-robin over the XCDs (workgroup L runs on XCD
// L % 8), so work items are handed out to give each XCD one contiguous range of
// them: the copies of a source then re-read it from the same L2.  The stores are
// non-temporal, which keeps the copies from evicting the sources there.  The
// step is bound by its writes; with both measures a fork of 1,792 pairs of
// 32 KiB blocks takes 23 us, against 39 us in plain pair order.
typedef unsigned CopyUnit __attribute__((ext_vector_type(4)));   // 16 B

__global__ __launch_bounds__(kCopyThreads) void kv_copy_blocks_kernel(CopyBlocksParams p) {
  const uint32_t n = p.work_items, L = blockIdx.x;
  const uint32_t q = n / kXcds, rem = n % kXcds, xcd = L % kXcds;
  const uint32_t w = xcd * q + min(xcd, rem) + L / kXcds;   // XCD x: [x q + min(x, rem), +q + (x < rem))
  const int pair = (int)(w / (uint32_t)p.slices);
  const int slice = (int)(w % (uint32_t)p.slices);
  const int src = p.src[pair];
  const int dst = p.dst[pair];
  if ((unsigned)src >= (unsigned)p.num_blocks || (unsigned)dst >= (unsigned)p.num_blocks ||
      src == dst)
    return;
  const int64_t off = (int64_t)slice * kCopySliceBytes + (int64_t)threadIdx.x * 16;
  if (off < p.block_bytes) {
    const uint4 kv = *reinterpret_cast<const uint4*>(p.k_cache + (size_t)src * p.block_bytes + off);
    const uint4 vv = *reinterpret_cast<const uint4*>(p.v_cache + (size_t)src * p.block_bytes + off);
    __builtin_nontemporal_store(__builtin_bit_cast(CopyUnit, kv),
                                reinterpret_cast<CopyUnit*>(p.k_cache + (size_t)dst * p.block_bytes + off));
    __builtin_nontemporal_store(__builtin_bit_cast(CopyUnit, vv),
                                reinterpret_cast<CopyUnit*>(p.v_cache + (size_t)dst * p.block_bytes + off));
  }
  if (p.k_scale && slice == 0) {
    for (int h = threadIdx.x; h < p.k_scales; h += kCopyThreads)
      p.k_scale[(size_t)dst * p.k_scales + h] = p.k_scale[(size_t)src * p.k_scales + h];
    for (int h = threadIdx.x; h < p.v_scales; h += kCopyThreads)
      p.v_scale[(size_t)dst * p.v_scales + h] = p.v_scale[(size_t)src * p.v_scales + h];
  }
}

struct GatherParams {
  const char* cache;            // [NB][Hkv][BS][row_bytes]
  const int32_t* block_table;   // row of the sequence
  char* out;                    // [Hkv][num_tokens][row_bytes]
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t num_blocks;
  int32_t num_tokens;
  int32_t row_bytes;            // head_dim * element size (multiple of 16)
};

// grid: (ceil(num_tokens / 64), Hkv); 256 threads copy 16 B units of 64 rows.
__global__ __launch_bounds__(256) void kv_gather_kernel(GatherParams p) {
  const int h = blockIdx.y;
  const int upr = p.row_bytes / 16;
  const int t0 = blockIdx.x * 64;
  for (int u = threadIdx.x; u < 64 * upr; u += blockDim.x) {
    const int t = t0 + u / upr;
    const int c = u % upr;
    if (t >= p.num_tokens) continue;
    const int blk = p.block_table[t / p.block_size];
    if (blk < 0 || blk >= p.num_blocks) continue;
    const size_t src = (((size_t)blk * p.num_kv_heads + h) * p.block_size + t % p.block_size) *
                           (size_t)p.row_bytes + (size_t)c * 16;
    const size_t dst = ((size_t)h * p.num_tokens + t) * (size_t)p.row_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(p.out + dst) = *reinterpret_cast<const uint4*>(p.cache + src);
  }
}

}  // namespace gqa
