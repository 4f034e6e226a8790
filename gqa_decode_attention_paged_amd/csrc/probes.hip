// Host side of the read-bandwidth probes (include/gqa_probe.h).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

#include "gqa_probe.h"
#include "probes.h"

namespace {

template <int POLICY>
const void* pick(int tile_bytes) {
  switch (tile_bytes) {
    case 1024: return reinterpret_cast<const void*>(&gqa::probe_read_kernel<1024, POLICY>);
    case 2048: return reinterpret_cast<const void*>(&gqa::probe_read_kernel<2048, POLICY>);
    case 4096: return reinterpret_cast<const void*>(&gqa::probe_read_kernel<4096, POLICY>);
    case 8192: return reinterpret_cast<const void*>(&gqa::probe_read_kernel<8192, POLICY>);
    case 16384: return reinterpret_cast<const void*>(&gqa::probe_read_kernel<16384, POLICY>);
  }
  return nullptr;
}

}  // namespace

extern "C" gqa_status gqa_probe_read(const void* pool, int64_t pool_tiles, const int32_t* tile_ids,
                                     int64_t num_tiles, int32_t tile_bytes, int32_t non_temporal,
                                     int32_t num_workgroups, uint32_t* sink, hipStream_t stream) {
  const void* fn = non_temporal ? pick<2>(tile_bytes) : pick<0>(tile_bytes);
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
