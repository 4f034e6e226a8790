// Host side of the read-bandwidth probes (include/gqa_probe.h).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

#include "gqa_probe.h"
#include "probes.h"

static_assert(gqa::kProbeWholeRows == GQA_PROBE_WHOLE_ROWS &&
                  gqa::kProbeOperandRows256 == GQA_PROBE_OPERAND_ROWS_256 &&
                  gqa::kProbeOperandRows128 == GQA_PROBE_OPERAND_ROWS_128 &&
                  gqa::kProbeOperandRows128Narrow == GQA_PROBE_OPERAND_ROWS_128_NARROW &&
                  gqa::kProbeMixed256 == GQA_PROBE_MIXED_256,
              "probe patterns match the header");

namespace {

template <int POLICY, int PATTERN>
const void* pick_tile(int tile_bytes) {
  switch (tile_bytes) {
#define GQA_PROBE_TILE(T)                                                             \
  case T:                                                                             \
    if constexpr (gqa::probe_pattern_fits(PATTERN, T))                                \
      return reinterpret_cast<const void*>(&gqa::probe_read_kernel<T, POLICY, PATTERN>); \
    return nullptr;
    GQA_PROBE_TILE(1024)
    GQA_PROBE_TILE(2048)
    GQA_PROBE_TILE(4096)
    GQA_PROBE_TILE(8192)
    GQA_PROBE_TILE(16384)
#undef GQA_PROBE_TILE
  }
  return nullptr;
}

template <int POLICY>
const void* pick(int tile_bytes, int pattern) {
  switch (pattern) {
    case gqa::kProbeWholeRows: return pick_tile<POLICY, gqa::kProbeWholeRows>(tile_bytes);
    case gqa::kProbeOperandRows256: return pick_tile<POLICY, gqa::kProbeOperandRows256>(tile_bytes);
    case gqa::kProbeOperandRows128: return pick_tile<POLICY, gqa::kProbeOperandRows128>(tile_bytes);
    case gqa::kProbeOperandRows128Narrow:
      return pick_tile<POLICY, gqa::kProbeOperandRows128Narrow>(tile_bytes);
    case gqa::kProbeMixed256: return pick_tile<POLICY, gqa::kProbeMixed256>(tile_bytes);
  }
  return nullptr;
}

}  // namespace

extern "C" gqa_status gqa_probe_read_pattern(const void* pool, int64_t pool_tiles,
                                             const int32_t* tile_ids, int64_t num_tiles,
                                             int32_t tile_bytes, int32_t pattern,
                                             int32_t non_temporal, int32_t num_workgroups,
                                             uint32_t* sink, hipStream_t stream) {
  const void* fn = non_temporal ? pick<2>(tile_bytes, pattern) : pick<0>(tile_bytes, pattern);
  if (!fn) return GQA_ERR_UNSUPPORTED;
  if (!pool || !sink || pool_tiles < 1 || num_tiles < 0 || num_workgroups < 1 ||
      num_workgroups > (1 << 20) || (reinterpret_cast<uintptr_t>(pool) & 15u) != 0)
    return GQA_ERR_INVALID_ARG;
  if (!tile_ids && num_tiles > pool_tiles) return GQA_ERR_INVALID_ARG;
  if (num_tiles == 0) return GQA_OK;
  const char* p = static_cast<const char*>(pool);
  int64_t per_wg = (num_tiles + num_workgroups - 1) / num_workgroups;
  void* args[] = {&p, &pool_tiles, &tile_ids, &num_tiles, &per_wg, &sink};
  const hipError_t e = hipLaunchKernel(fn, dim3(num_workgroups), dim3(gqa::kProbeThreads), args, 0,
                                       stream);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

extern "C" gqa_status gqa_probe_read(const void* pool, int64_t pool_tiles, const int32_t* tile_ids,
                                     int64_t num_tiles, int32_t tile_bytes, int32_t non_temporal,
                                     int32_t num_workgroups, uint32_t* sink, hipStream_t stream) {
  return gqa_probe_read_pattern(pool, pool_tiles, tile_ids, num_tiles, tile_bytes,
                                gqa::kProbeWholeRows, non_temporal, num_workgroups, sink, stream);
}
