/*
 * gqa_probe.h — read-bandwidth probes of libgqa_paged.so (measurement only; not
 * on the decode path).
 *
 * The decode step is bound by reading the KV cache once (*The Mathematics of
 * Transformer Inference* (hs-black) §4 and §6: the step's lower bound is the
 * time to read the cache at the memory bandwidth).  Peak and sustained
 * bandwidth are different figures, and the sustained one is measured with a
 * microbenchmark of the same access pattern (*LLM Inference Systems
 * Engineering* (jasonzhang109) §3.8.2).  This probe is that microbenchmark: it
 * reads tiles exactly as the decode kernel reads its (block, KV head) tiles,
 * with no compute, no merge and no append, so its rate is the ceiling the
 * decode kernel's KV-read rate is compared with.
 */
#ifndef GQA_PROBE_H
#define GQA_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "gqa_paged.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gqa_probe_read — one launch that reads num_tiles tiles of tile_bytes bytes.
 *   pool          device buffer of pool_tiles * tile_bytes bytes, 16-byte aligned
 *   tile_ids      [num_tiles] int32 device array: tile t is read at
 *                 pool + tile_ids[t] * tile_bytes (ids outside [0, pool_tiles)
 *                 read tile 0); NULL reads tile t at pool + t * tile_bytes
 *                 (a plain streaming read; then num_tiles <= pool_tiles)
 *   tile_bytes    1024, 2048, 4096, 8192 or 16384 (the (block, KV head) tile of
 *                 the pools: block_size * head_dim * element bytes)
 *   non_temporal  1: loads carry the non-temporal cache-policy hint, as the
 *                 decode kernel's K/V tile loads do; 0: default policy
 *   num_workgroups  workgroups of 8 waves (the decode kernel's), one per compute
 *                 unit for the full-chip figure, 1 for a lone workgroup; each
 *                 takes a contiguous range of the table, its waves interleaved
 *                 groups of 16 KiB of tiles
 *   sink          [num_workgroups * 8] uint32 device array receiving a checksum
 *                 per wave (written; keeps the loads live)
 * Asynchronous on `stream`.  GQA_ERR_INVALID_ARG / GQA_ERR_UNSUPPORTED for bad
 * host arguments, GQA_ERR_HIP when the launch fails.
 */
gqa_status gqa_probe_read(const void* pool, int64_t pool_tiles, const int32_t* tile_ids,
                          int64_t num_tiles, int32_t tile_bytes, int32_t non_temporal,
                          int32_t num_workgroups, uint32_t* sink, hipStream_t stream);

/*
 * Per-instruction load patterns: how the 64 lanes of one wave load instruction
 * cover a tile, in the ways the decode kernel reads its tiles.  Every pattern
 * reads each 32-bit word of a tile exactly once.
 */
enum {
  GQA_PROBE_WHOLE_ROWS = 0,           /* 16 B per lane, 1 KiB contiguous per
                                         instruction (V rows; K rows on the vector
                                         path, and on the matrix path at 16 rows
                                         or more) */
  GQA_PROBE_OPERAND_ROWS_256 = 1,     /* 16 rows x 64 B of 256-byte rows, 16 B per
                                         lane: bf16 K (d_h 128) loaded straight
                                         into the MFMA operand layout */
  GQA_PROBE_OPERAND_ROWS_128 = 2,     /* 16 rows x 64 B of 128-byte rows, 16 B per
                                         lane: fp8 K (d_h 128) in the operand
                                         layout, two score steps per lane */
  GQA_PROBE_OPERAND_ROWS_128_NARROW = 3,  /* 16 rows x 32 B of 128-byte rows, 8 B per
                                         lane: fp8 K with one score step per lane */
  GQA_PROBE_MIXED_256 = 4             /* even table entries as OPERAND_ROWS_256,
                                         odd ones as WHOLE_ROWS: the K and V tiles
                                         of a bf16 step */
};

/*
 * gqa_probe_read_pattern — gqa_probe_read with the per-instruction load
 * pattern `pattern` (GQA_PROBE_*); gqa_probe_read is GQA_PROBE_WHOLE_ROWS.
 * tile_bytes must be a multiple of 4096 for OPERAND_ROWS_256 and MIXED_256
 * and of 2048 for the 128-byte-row patterns; other sizes and patterns return
 * GQA_ERR_UNSUPPORTED.  Arguments and errors are otherwise gqa_probe_read's.
 */
gqa_status gqa_probe_read_pattern(const void* pool, int64_t pool_tiles, const int32_t* tile_ids,
                                  int64_t num_tiles, int32_t tile_bytes, int32_t pattern,
                                  int32_t non_temporal, int32_t num_workgroups, uint32_t* sink,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBE_H */
