// Read-bandwidth probes: the ceiling the decode kernel's KV reads are measured
// against.  A probe launch reads `num_tiles` tiles of TILE contiguous bytes,
// tile t at pool + ids[t] * TILE (or t * TILE without a table), and does
// nothing else with them but fold them into a checksum: no compute, no merge.
// With a random table and the tile size of a (block, KV head) tile it is the
// paged gather of the decode step; with no table it is a plain streaming read.
//
// The access pattern copies the decode kernel's: 8-wave workgroups, one per
// compute unit; waves take interleaved groups of tiles; each lane reads 16 bytes
// per load through a buffer resource whose base is the tile (scalar registers);
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

template <int TILE, int POLICY>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(
    const char* __restrict__ pool, int64_t pool_tiles, const int32_t* __restrict__ ids,
    int64_t num_tiles, int64_t tiles_per_wg, uint32_t* __restrict__ sink) {
  static_assert(TILE % 1024 == 0 && TILE <= kProbeInFlight, "tile of whole wave loads");
  constexpr int kWaves = kProbeThreads / kWave;
  constexpr int NL = TILE / 1024;                         // 16-byte loads per lane per tile
  constexpr int U = kProbeInFlight / TILE;               // tiles per wave per round
  const int lane = threadIdx.x & (kWave - 1);
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
#pragma unroll
      for (int l = 0; l < NL; ++l)
        v[u][l] = in ? __builtin_bit_cast(probe_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rsrc, lane * 16 + l * 1024, 0,
                                                           POLICY))
                     : probe_u32x4{0u, 0u, 0u, 0u};
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
