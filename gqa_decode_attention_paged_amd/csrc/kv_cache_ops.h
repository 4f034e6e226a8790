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
// All are plain byte copies in 16-byte units (bit-exact).
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

struct CopyBlocksParams {
  char* k_cache;                // [NB][Hkv][BS][row_bytes]
  char* v_cache;
  float* k_scale;               // [NB][Hkv] fp8 scales, or null
  float* v_scale;
  const int32_t* src;           // [num_pairs] source block ids
  const int32_t* dst;           // [num_pairs] destination block ids
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t tile_bytes;           // BS * row_bytes, a multiple of 16
};

// grid: (num_pairs, Hkv); 256 threads copy one (block, KV head) tile of K and
// of V.  Pairs with an id outside the pool, or src == dst, copy nothing.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(CopyBlocksParams p) {
  const int src = p.src[blockIdx.x];
  const int dst = p.dst[blockIdx.x];
  if ((unsigned)src >= (unsigned)p.num_blocks || (unsigned)dst >= (unsigned)p.num_blocks ||
      src == dst)
    return;
  const size_t h = blockIdx.y;
  const size_t so = ((size_t)src * p.num_kv_heads + h) * p.tile_bytes;
  const size_t dof = ((size_t)dst * p.num_kv_heads + h) * p.tile_bytes;
  for (int u = threadIdx.x; u < p.tile_bytes / 16; u += blockDim.x) {
    *reinterpret_cast<uint4*>(p.k_cache + dof + (size_t)u * 16) =
        *reinterpret_cast<const uint4*>(p.k_cache + so + (size_t)u * 16);
    *reinterpret_cast<uint4*>(p.v_cache + dof + (size_t)u * 16) =
        *reinterpret_cast<const uint4*>(p.v_cache + so + (size_t)u * 16);
  }
  if (p.k_scale && threadIdx.x == 0) {
    p.k_scale[(size_t)dst * p.num_kv_heads + h] = p.k_scale[(size_t)src * p.num_kv_heads + h];
    p.v_scale[(size_t)dst * p.num_kv_heads + h] = p.v_scale[(size_t)src * p.num_kv_heads + h];
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
