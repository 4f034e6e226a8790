// Read-bandwidth probes: the ceiling the decode kernel's KV reads are measured
// against.  A probe launch reads `num_tiles` tiles of TILE contiguous bytes,
// tile t at pool + ids[t] * TILE (or t * TILE without a table), and does
// nothing else with them but fold them into a checksum: no compute, no merge.
// With a random table and the tile size of a (block, KV head) tile it is the
// paged gather of the decode step; with no table it is a plain streaming read.
//
// The access pattern copies the decode kernel's: 8-wave workgroups, one per
// compute unit; waves take interleaved groups of tiles; each lane reads 16 (or
// 8) bytes per load, in one of the decode kernel's per-instruction patterns
// (ProbePattern), through a buffer resource whose base is the tile (scalar registers);
// every wave keeps kProbeInFlight bytes of loads in flight, as the decode
// kernel keeps the next chunk's K and V rows (32 tokens x 2 x 256 bytes) in
// flight.  The load cache policy is a template parameter (default, or the
// non-temporal hint the decode kernel uses).
#pragma once

#include "common.h"

namespace gqa {

constexpr int kProbeThreads = 512;                 // 8 waves
constexpr int kProbeInFlight = 16384;              // bytes of loads in flight per wave

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

// How each wave instruction covers a tile (the ways the decode kernel reads one):
//  kProbeWholeRows      64 lanes x 16 B, contiguous: 1 KiB of whole rows (V rows,
//                       and K rows on the vector path);
//  kProbeOperandRows256 16 rows x 64 B of 256-byte rows, 16 B per lane: bf16 K
//                       loaded straight into the MFMA operand layout (d_h 128);
//  kProbeOperandRows128 16 rows x 64 B of 128-byte rows, 16 B per lane: fp8 K in
//                       the operand layout, two score steps per lane;
//  kProbeOperandRows128Narrow  16 rows x 32 B of 128-byte rows, 8 B per lane:
//                       fp8 K in the operand layout, one score step per lane;
//  kProbeMixed256       even table entries as kProbeOperandRows256, odd ones as
//                       kProbeWholeRows (K and V tiles of a bf16 step).
// Every pattern reads each 32-bit word of a tile exactly once.
enum ProbePattern {
  kProbeWholeRows = 0,
  kProbeOperandRows256 = 1,
  kProbeOperandRows128 = 2,
  kProbeOperandRows128Narrow = 3,
  kProbeMixed256 = 4,
  kProbePatterns = 5
};

__host__ __device__ constexpr bool probe_pattern_fits(int pattern, int tile) {
  return pattern == kProbeWholeRows ? tile % 1024 == 0
         : (pattern == kProbeOperandRows256 || pattern == kProbeMixed256) ? tile % 4096 == 0
                                                                           : tile % 2048 == 0;
}

template <int TILE, int POLICY, int PATTERN>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(
    const char* __restrict__ pool, int64_t pool_tiles, const int32_t* __restrict__ ids,
    int64_t num_tiles, int64_t tiles_per_wg, uint32_t* __restrict__ sink) {
  static_assert(TILE <= kProbeInFlight && probe_pattern_fits(PATTERN, TILE), "tile geometry");
  constexpr int kWaves = kProbeThreads / kWave;
  constexpr int LB = PATTERN == kProbeOperandRows128Narrow ? 8 : 16;   // bytes per lane per load
  constexpr int NL = TILE / (kWave * LB);                 // loads per lane per tile
  constexpr int U = kProbeInFlight / TILE;               // tiles per wave per round
  const int lane = threadIdx.x & (kWave - 1);
  const int hd = lane & 15, qd = lane >> 4;               // operand layout: row, lane group
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t first = (int64_t)blockIdx.x * tiles_per_wg;
  const int64_t last = first + tiles_per_wg < num_tiles ? first + tiles_per_wg : num_tiles;
  uint32_t acc = 0;
  for (int64_t t0 = first + (int64_t)wave * U; t0 < last; t0 += (int64_t)kWaves * U) {
    probe_u32x4 v[U][NL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u;
      const bool in = t < last;
      int64_t id = in ? (ids ? (int64_t)ids[t] : t) : 0;
      id = id >= 0 && id < pool_tiles ? id : 0;
      const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(pool) + id * TILE, 0,
                                                          TILE, 0x00020000);
      const bool operand = PATTERN == kProbeMixed256 ? (t & 1) == 0 : PATTERN != kProbeWholeRows;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        int off;
        if constexpr (PATTERN == kProbeOperandRows128)
          off = ((l / 2) * 16 + hd) * 128 + (l % 2) * 64 + qd * 16;
        else if constexpr (PATTERN == kProbeOperandRows128Narrow)
          off = ((l / 4) * 16 + hd) * 128 + (l % 4) * 32 + qd * 8;
        else
          off = operand ? ((l / 4) * 16 + hd) * 256 + (l % 4) * 64 + qd * 16 : lane * 16 + l * 1024;
        if constexpr (LB == 8) {
          const uint2 w = in ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                             rsrc, off, 0, POLICY))
                             : make_uint2(0u, 0u);
          v[u][l] = probe_u32x4{w.x, w.y, 0u, 0u};
        } else {
          v[u][l] = in ? __builtin_bit_cast(probe_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             rsrc, off, 0, POLICY))
                       : probe_u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int l = 0; l < NL; ++l) acc ^= v[u][l].x ^ v[u][l].y ^ v[u][l].z ^ v[u][l].w;
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) acc ^= __shfl_xor(acc, m, kWave);
  if (lane == 0) sink[(size_t)blockIdx.x * kWaves + wave] = acc;
}

}  // namespace gqa
