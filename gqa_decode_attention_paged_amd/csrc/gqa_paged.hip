// Host side of the paged GQA decode-attention library: argument validation,
// workspace sizing, kernel selection and launches.  The C ABI is declared in
// include/gqa_paged.h; the device code lives in the headers next to this file.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "gqa_paged.h"
#include "common.h"
#include "decode_kernel.h"
#include "kv_cache_ops.h"


namespace {

thread_local std::string g_last_error;


gqa_status fail(gqa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gqa_status ok() {
  g_last_error.clear();
  return GQA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point.
gqa_status check_shape(const gqa_paged_shape* s) {
  if (!s) return fail(GQA_ERR_INVALID_ARG, "shape is NULL");
  if (s->num_seqs < 0) return fail(GQA_ERR_INVALID_ARG, "num_seqs %d < 0", s->num_seqs);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(GQA_ERR_INVALID_ARG, "head counts must be >= 1 (H_q=%d, H_kv=%d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(GQA_ERR_INVALID_ARG, "H_q=%d is not a multiple of H_kv=%d", s->num_q_heads,
                s->num_kv_heads);
  if (s->num_blocks < 1 || s->max_blocks_per_seq < 1)
    return fail(GQA_ERR_INVALID_ARG, "num_blocks=%d and max_blocks_per_seq=%d must be >= 1",
                s->num_blocks, s->max_blocks_per_seq);
  if (s->head_dim < 1 || s->block_size < 1)
    return fail(GQA_ERR_INVALID_ARG, "head_dim and block_size must be >= 1");
  const int G = s->num_q_heads / s->num_kv_heads;
  // A KV head's rows (G per query position) map to heads by shift and mask, and
  // the kernels take at most 32 of them (checked per call, with the positions).
  if (G > 32 || (G & (G - 1)) != 0)
    return fail(GQA_ERR_UNSUPPORTED, "group size G=%d not in {1,2,4,8,16,32}", G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(GQA_ERR_UNSUPPORTED, "head_dim=%d not in {64,128}", s->head_dim);
  if (s->block_size != 16 && s->block_size != 32)
    return fail(GQA_ERR_UNSUPPORTED, "block_size=%d not in {16,32}", s->block_size);
  if (s->kv_dtype != GQA_KV_BF16 && s->kv_dtype != GQA_KV_FP8_E4M3 &&
      s->kv_dtype != GQA_KV_FP8_E4M3_KIVI)
    return fail(GQA_ERR_UNSUPPORTED, "kv_dtype=%d unknown", s->kv_dtype);
  if (s->flags & ~GQA_FLAG_BATCH_INVARIANT)
    return fail(GQA_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)s->flags);
  if (s->sliding_window < 0)
    return fail(GQA_ERR_INVALID_ARG, "sliding_window %d < 0", s->sliding_window);
  if ((int64_t)s->max_blocks_per_seq * s->block_size > INT32_MAX)
    return fail(GQA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size overflows int32");
  return GQA_OK;
}

struct WorkspaceLayout {
  size_t o_off, lse_off, cnt_words, total;
};

// Rows per (sequence, KV head): G * Q, rounded up to a power of two (the
// kernel's row capacity M).
int row_capacity(int rows) {
  int m = 1;
  while (m < rows) m <<= 1;
  return m;
}

// [counters: B*Hkv*kCounterStride u32][partial outputs: B*Hkv*S*M*D fp32]
// [partial lse: B*Hkv*S*M fp32].  The counters come first so that a workspace
// initialised for one shape serves any later call with no more (sequence, KV
// head) pairs.
WorkspaceLayout workspace_layout(const gqa_paged_shape* s, int max_splits, int num_queries) {
  WorkspaceLayout w;
  w.cnt_words = (size_t)s->num_seqs * s->num_kv_heads * gqa::kCounterStride;
  const int G = s->num_q_heads / s->num_kv_heads;
  const size_t rows = (size_t)s->num_seqs * s->num_kv_heads *
                      (size_t)row_capacity(G * num_queries) * (size_t)max_splits;
  w.o_off = (w.cnt_words * sizeof(uint32_t) + 255) & ~size_t(255);
  w.lse_off = (w.o_off + rows * s->head_dim * sizeof(float) + 255) & ~size_t(255);
  w.total = w.lse_off + rows * sizeof(float);
  return w;
}

// Splits a launch or a workspace must provide for every attended length up to
// `len` under target `target`: a split plan never uses more than
// min(target, ceil(len / kMinSplitTokens)), while the plan of `len` itself may
// round to fewer than a shorter length's plan.
int split_bound(int64_t len, int target, int min_tokens = gqa::kMinSplitTokens) {
  const int64_t n = (len + min_tokens - 1) / min_tokens;
  const int64_t b = n < target ? n : target;
  return b < 1 ? 1 : (int)b;
}

int max_splits_for(int32_t max_context_len) { return split_bound(max_context_len, gqa::kMaxSplits); }

// Longest attended span any sequence can have: the whole hint, or with a
// sliding window the window plus the other query positions plus the partial
// block the span starts in.
int64_t max_span(const gqa_paged_shape* s, int32_t max_context_len, int32_t num_queries) {
  if (s->sliding_window <= 0) return max_context_len;
  const int64_t w = (int64_t)s->sliding_window + num_queries - 1 + s->block_size - 1;
  return w < max_context_len ? w : max_context_len;
}

// Kernel dispatch over the supported (D, BS, rows M, dtype, waves) combinations.
// M is the row capacity, the power of two at or above G * Q: up to 32 on the
// matrix path (bf16 pools and fp8 pools with per-(block, head) scales; 32 rows
// are two row tiles and run on 4-wave workgroups only), up to 8 for KIVI pools
// (vector path).
constexpr int kMaxRows = 32;
constexpr int kMaxRowsKivi = 8;

// kv: 0 bf16, 1 fp8 with (block, KV head) scales, 2 fp8 with the KIVI layout.
template <int D, int BS, int M, int W>
const void* pick_kernel_m(int kv) {
  if constexpr (M > 16 && W != 4) {
    return nullptr;
  } else if constexpr (M > kMaxRowsKivi) {
    switch (kv) {
      case 0: return reinterpret_cast<const void*>(&gqa::paged_decode_kernel<D, BS, M, 0, W>);
      case 1: return reinterpret_cast<const void*>(&gqa::paged_decode_kernel<D, BS, M, 1, W>);
    }
    return nullptr;
  } else {
    switch (kv) {
      case 0: return reinterpret_cast<const void*>(&gqa::paged_decode_kernel<D, BS, M, 0, W>);
      case 1: return reinterpret_cast<const void*>(&gqa::paged_decode_kernel<D, BS, M, 1, W>);
      case 2: return reinterpret_cast<const void*>(&gqa::paged_decode_kernel<D, BS, M, 2, W>);
    }
    return nullptr;
  }
}

template <int D, int BS, int W>
const void* pick_kernel_bs(int M, int fp8) {
  switch (M) {
    case 1: return pick_kernel_m<D, BS, 1, W>(fp8);
    case 2: return pick_kernel_m<D, BS, 2, W>(fp8);
    case 4: return pick_kernel_m<D, BS, 4, W>(fp8);
    case 8: return pick_kernel_m<D, BS, 8, W>(fp8);
    case 16: return pick_kernel_m<D, BS, 16, W>(fp8);
    case 32: return pick_kernel_m<D, BS, 32, W>(fp8);
  }
  return nullptr;
}

template <int W>
const void* pick_kernel_w(int D, int BS, int M, int fp8) {
  if (D == 64)
    return BS == 16 ? pick_kernel_bs<64, 16, W>(M, fp8) : pick_kernel_bs<64, 32, W>(M, fp8);
  return BS == 16 ? pick_kernel_bs<128, 16, W>(M, fp8) : pick_kernel_bs<128, 32, W>(M, fp8);
}

const void* pick_kernel(int D, int BS, int M, int fp8, int waves) {
  return waves == 8 ? pick_kernel_w<8>(D, BS, M, fp8) : pick_kernel_w<4>(D, BS, M, fp8);
}


// Waves per workgroup.  An eight-wave workgroup covers twice the tokens of a
// four-wave one at the same number of resident waves (one per CU instead of
// two), so each (sequence, KV head) has half as many splits to publish, count
// and merge.  Batch-invariant calls use four-wave workgroups over the fixed
// 64-split plan, whose shortest splits (128 tokens) fill four waves.
//
// A batch of several sequences whose eight-wave plan gives each at most two
// splits takes four-wave workgroups too: twice the slots to share out by
// length.  On 16 sequences of 512-8192 tokens (8 KV heads) that is 49.6 against
// 51.9 us; the same shape with equal lengths, where the sharing has nothing to
// balance, gives back 1% (48.2 against 47.7 us).  The lengths live on the
// device, so the host cannot tell the two apart.
int target_splits(const gqa_paged_shape* s, const void* fn, int threads, bool invariant);

// Tuning overrides, read once from the environment (unset or invalid: the
// defaults): GQA_WAVES = 4 or 8 waves per workgroup; GQA_SPLIT_ROUNDS = r > 0
// sizes the split target for r rounds of the resident-workgroup capacity.
// Neither applies to batch-invariant calls.  Results change in the last bits
// with either, as with any other split plan.
int env_override(const char* name, int lo, int hi) {
  const char* v = getenv(name);
  if (!v || !*v) return 0;
  char* end = nullptr;
  const long x = strtol(v, &end, 10);
  return (*end == 0 && x >= lo && x <= hi) ? (int)x : 0;
}
int waves_override() {
  static const int w = [] {
    const int x = env_override("GQA_WAVES", 4, 8);
    return x == 4 || x == 8 ? x : 0;
  }();
  return w;
}
int rounds_override() {
  static const int r = env_override("GQA_SPLIT_ROUNDS", 1, 64);
  return r;
}
// GQA_DEFER_MERGE: 1 merges the splits in merge_splits_kernel after the decode
// launch, 2 in the decode launch's last workgroup; unset, the library chooses
// (below).
int defer_merge_override() {
  static const int d = env_override("GQA_DEFER_MERGE", 1, 2);
  return d;
}

// Split-length override (GQA_SPLIT_TOKENS, or gqa_set_split_tokens at run time):
// 0, or the shortest split in tokens, a multiple of kChunkTokens in
// [kMinSplitTokens, kMaxSplitTokensOverride].  When set, every attention call
// takes the batch-invariant plan with that minimum in place of kMinSplitTokens.
constexpr int kMaxSplitTokensOverride = 1 << 19;   // T / 32 fits the kernel's 15 plan bits
bool valid_split_tokens(int t) {
  return t >= gqa::kMinSplitTokens && t <= kMaxSplitTokensOverride && t % gqa::kChunkTokens == 0;
}
std::atomic<int>& split_tokens_setting() {
  static std::atomic<int> v{[] {
    const int x = env_override("GQA_SPLIT_TOKENS", gqa::kMinSplitTokens, kMaxSplitTokensOverride);
    return valid_split_tokens(x) ? x : 0;
  }()};
  return v;
}

int resident_workgroups(const void* fn, int threads);

// Waves per workgroup, and the waves of the variant whose resident capacity
// sizes the split target (the same, except for one four-wave workgroup per CU).
struct WavePlan {
  int waves;
  int target_waves;
};

WavePlan pick_waves(const gqa_paged_shape* s, int row_cap, int kv, bool fused_append,
                    bool invariant) {
  if (row_cap > 16) return {4, 4};     // two row tiles: one 4-wave workgroup per CU
  if (invariant) return {4, 4};
  if (waves_override()) return {waves_override(), waves_override()};
  const void* fn8 = pick_kernel(s->head_dim, s->block_size, row_cap, kv, 8);
  const void* fn4 = pick_kernel(s->head_dim, s->block_size, row_cap, kv, 4);
  if (!fn8) return {4, 4};
  if (s->num_seqs >= 2 && target_splits(s, fn8, 8 * 64, false) <= 2) return {4, 4};
  // More resident waves with four-wave workgroups: a variant whose registers
  // allow an odd number of waves per SIMD (the fp8 single-row variant fits 5)
  // leaves one idle under eight-wave workgroups.  On the 40-head fp8 MHA
  // workload that is 56.2 against 57.6 us; where the counts tie, eight waves
  // keep half as many partials to merge.  The same step with the fused
  // quantising append measured the other way (59.8 against 58.0 us), so it
  // keeps eight.
  if (!fused_append && fn4 &&
      (int64_t)resident_workgroups(fn4, 4 * 64) * 4 >
          (int64_t)resident_workgroups(fn8, 8 * 64) * 8)
    return {4, 4};
  // One four-wave workgroup per CU, at the eight-wave split count, where the
  // matrix path's work per byte is light: bf16 up to 8 rows, fp8 (whose codes
  // are widened first) up to 4.  Four waves stream as fast as eight there, and
  // the workgroup has half as many waves to start and to merge: 8K, G = 4:
  // 13.2 against 13.9 us; 32K, G = 8: 85.3 against 86.1; fp8 8K, G = 4: 12.3
  // against 12.5.  Heavier rows need the second wave per SIMD to hide their
  // compute: fp8 32K, G = 8: 70.9 against 62.9 us; 16 rows (8K, 4 positions,
  // G = 4): 20.5 against 18.1.
  const bool matrix = kv != 2 && row_cap >= 2;
  if (matrix && fn4 && row_cap * (kv == 1 ? 2 : 1) <= 8) return {4, 8};
  return {8, 8};
}

// Workgroups of `fn` the current device keeps resident at once (compute units
// times workgroups per unit at this kernel's register and LDS use); cached.
int resident_workgroups(const void* fn, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, fn});
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess)
    return 0;
  const int cap = cus * (per_cu > 0 ? per_cu : 1);
  cache[{dev, fn}] = cap;
  return cap;
}

// Split-count target.  By default, as many splits as let the batch's (sequence,
// KV head) pairs fill the resident-workgroup capacity once without exceeding
// it (fewer, longer splits amortise each workgroup's start-up and merge, and a
// partial second round of workgroups would only add a tail).  With
// GQA_FLAG_BATCH_INVARIANT or a split-length override, the fixed maximum, so
// the split of a sequence depends on its own length only.
int target_splits(const gqa_paged_shape* s, const void* fn, int threads, bool invariant) {
  if (invariant) return gqa::kMaxSplits;
  const int cap = resident_workgroups(fn, threads);
  if (cap <= 0) return gqa::kMaxSplits;
  const int64_t pairs = (int64_t)s->num_seqs * s->num_kv_heads;
  const int rounds = rounds_override() ? rounds_override() : 1;
  int64_t t = (int64_t)rounds * cap / pairs;   // one round: never more workgroups than fit
  if (t < 1) t = 1;
  if (t > gqa::kMaxSplits) t = gqa::kMaxSplits;
  return (int)t;
}

gqa_status launch(const void* fn, dim3 grid, dim3 block, void* params, const char* what,
                  hipStream_t stream) {
  void* args[] = {params};
  hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return GQA_OK;
}

}  // namespace

extern "C" {

const char* gqa_last_error(void) { return g_last_error.c_str(); }

const char* gqa_version(void) { return "gqa_paged 0.3 (gfx950)"; }

int32_t gqa_decode_num_splits(int32_t context_len) {
  const int t = split_tokens_setting().load(std::memory_order_relaxed);
  return gqa::split_plan(context_len, gqa::kMaxSplits, t > 0 ? t : gqa::kMinSplitTokens).num_splits;
}

gqa_status gqa_set_split_tokens(int32_t tokens) {
  if (tokens != 0 && !valid_split_tokens(tokens))
    return fail(GQA_ERR_INVALID_ARG,
                "split length %d: 0, or a multiple of %d in [%d, %d]", tokens, gqa::kChunkTokens,
                gqa::kMinSplitTokens, kMaxSplitTokensOverride);
  split_tokens_setting().store(tokens, std::memory_order_relaxed);
  return ok();
}

int32_t gqa_split_tokens(void) { return split_tokens_setting().load(std::memory_order_relaxed); }

size_t gqa_paged_decode_workspace_size(const gqa_paged_shape* shape, int32_t max_context_len) {
  if (check_shape(shape) != GQA_OK || max_context_len < 0) return 0;
  return workspace_layout(shape, split_bound(max_span(shape, max_context_len, 1), gqa::kMaxSplits),
                          1).total;
}

size_t gqa_paged_multi_query_workspace_size(const gqa_paged_shape* shape, int32_t num_queries,
                                            int32_t max_context_len) {
  if (check_shape(shape) != GQA_OK || max_context_len < 0 || num_queries < 1) return 0;
  return workspace_layout(shape,
                          split_bound(max_span(shape, max_context_len, num_queries), gqa::kMaxSplits),
                          num_queries).total;
}

static gqa_status append_impl(const gqa_paged_shape* s, int32_t num_tokens, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* positions,
                              hipStream_t stream) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535)
    return fail(GQA_ERR_INVALID_ARG, "num_tokens %d outside [0, 65535]", num_tokens);
  if (s->kv_dtype != GQA_KV_BF16)
    return fail(GQA_ERR_UNSUPPORTED,
                "kv_append copies bf16 rows; append to fp8 pools with gqa_kv_append_fp8");
  if (s->num_seqs == 0 || num_tokens == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !positions)
    return fail(GQA_ERR_INVALID_ARG, "kv_append: NULL device pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(GQA_ERR_INVALID_ARG, "kv_append: K/V pointers must be 16-byte aligned");
  gqa::AppendParams p;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.block_tables = block_tables;
  p.positions = positions;
  p.num_tokens = num_tokens;
  p.num_kv_heads = s->num_kv_heads;
  p.head_dim = s->head_dim;
  p.block_size = s->block_size;
  p.num_blocks = s->num_blocks;
  p.max_blocks = s->max_blocks_per_seq;
  st = launch(reinterpret_cast<const void*>(&gqa::kv_append_kernel),
              dim3(s->num_seqs, num_tokens), dim3(256), &p, "kv_append", stream);
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_kv_append(const gqa_paged_shape* s, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* block_tables,
                         const int32_t* positions, hipStream_t stream) {
  return append_impl(s, 1, k_new, v_new, k_cache, v_cache, block_tables, positions, stream);
}

gqa_status gqa_kv_append_tokens(const gqa_paged_shape* s, int32_t num_tokens, const void* k_new,
                                const void* v_new, void* k_cache, void* v_cache,
                                const int32_t* block_tables, const int32_t* positions,
                                hipStream_t stream) {
  return append_impl(s, num_tokens, k_new, v_new, k_cache, v_cache, block_tables, positions,
                     stream);
}

gqa_status gqa_kv_append_fp8(const gqa_paged_shape* s, int32_t num_tokens, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache, float* k_scale,
                             float* v_scale, const int32_t* block_tables,
                             const int32_t* start_positions, hipStream_t stream) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535)
    return fail(GQA_ERR_INVALID_ARG, "num_tokens %d outside [0, 65535]", num_tokens);
  if (s->kv_dtype == GQA_KV_BF16)
    return fail(GQA_ERR_INVALID_ARG, "kv_append_fp8 needs an fp8 pool (use kv_append for bf16)");
  const bool kivi = s->kv_dtype == GQA_KV_FP8_E4M3_KIVI;
  if (s->num_seqs == 0 || num_tokens == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables ||
      !start_positions)
    return fail(GQA_ERR_INVALID_ARG, "kv_append_fp8: NULL device pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(GQA_ERR_INVALID_ARG, "kv_append_fp8: K/V pointers must be 16-byte aligned");
  if (s->num_kv_heads > 65535)
    return fail(GQA_ERR_UNSUPPORTED, "kv_append_fp8: num_kv_heads %d > 65535", s->num_kv_heads);
  gqa::AppendFp8Params p;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_tables = block_tables;
  p.start = start_positions;
  p.num_tokens = num_tokens;
  p.num_kv_heads = s->num_kv_heads;
  p.head_dim = s->head_dim;
  p.block_size = s->block_size;
  p.num_blocks = s->num_blocks;
  p.max_blocks = s->max_blocks_per_seq;
  st = launch(kivi ? reinterpret_cast<const void*>(&gqa::kv_append_fp8_kivi_kernel)
                   : reinterpret_cast<const void*>(&gqa::kv_append_fp8_kernel),
              dim3(s->num_seqs, s->num_kv_heads, 2), dim3(256), &p, "kv_append_fp8", stream);
  return st == GQA_OK ? ok() : st;
}

static gqa_status decode_impl(const gqa_paged_shape* s, int32_t num_queries, const void* q,
                              void* k_cache,
                              void* v_cache, const float* k_scale, const float* v_scale,
                              const void* k_new, const void* v_new, const int32_t* positions,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t max_context_len, float softmax_scale, float* out,
                              float* out_lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, bool append_tail = false,
                              bool clear_counters = false) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (max_context_len < 0)
    return fail(GQA_ERR_INVALID_ARG, "max_context_len %d < 0", max_context_len);
  if ((int64_t)max_context_len > (int64_t)s->max_blocks_per_seq * s->block_size)
    return fail(GQA_ERR_INVALID_ARG, "max_context_len %d exceeds max_blocks_per_seq*block_size",
                max_context_len);
  if (!std::isfinite(softmax_scale))
    return fail(GQA_ERR_INVALID_ARG, "softmax_scale is not finite");
  const bool fp8 = s->kv_dtype != GQA_KV_BF16;
  const bool kivi = s->kv_dtype == GQA_KV_FP8_E4M3_KIVI;
  if (fp8 && (!k_scale || !v_scale))
    return fail(GQA_ERR_INVALID_ARG, "fp8 pools need k_scale and v_scale");
  const int64_t scales_per_tile = kivi ? (s->head_dim > s->block_size ? s->head_dim : s->block_size) : 1;
  if (fp8 && (int64_t)s->num_blocks * s->num_kv_heads * scales_per_tile * 4 > INT32_MAX)
    return fail(GQA_ERR_UNSUPPORTED, "fp8 scale arrays of %lld bytes exceed 2 GiB",
                (long long)s->num_blocks * s->num_kv_heads * scales_per_tile * 4);
  if (!fp8 && (k_scale || v_scale))
    return fail(GQA_ERR_INVALID_ARG, "k_scale/v_scale must be NULL for bf16 pools");
  const int G = s->num_q_heads / s->num_kv_heads;
  if (num_queries < 1) return fail(GQA_ERR_INVALID_ARG, "num_queries %d < 1", num_queries);
  if ((int64_t)G * num_queries > (kivi ? kMaxRowsKivi : kMaxRows))
    return fail(GQA_ERR_UNSUPPORTED, "G * num_queries = %lld rows exceeds %d for this KV dtype",
                (long long)G * num_queries, kivi ? kMaxRowsKivi : kMaxRows);
  const int rows = G * num_queries;
  if (append_tail && num_queries > s->block_size)
    return fail(GQA_ERR_UNSUPPORTED, "the fused append takes at most block_size (%d) tokens",
                s->block_size);
  if (s->num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(GQA_ERR_INVALID_ARG, "decode: NULL device pointer");
  if ((positions || append_tail) && (!k_new || !v_new))
    return fail(GQA_ERR_INVALID_ARG, "append: NULL k_new/v_new");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
    return fail(GQA_ERR_INVALID_ARG, "decode: q, caches, new rows and out must be 16-byte aligned");
  const int ws_splits = split_bound(max_span(s, max_context_len, num_queries), gqa::kMaxSplits);
  const WorkspaceLayout wl = workspace_layout(s, ws_splits, num_queries);
  if (!workspace || workspace_bytes < wl.total)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                wl.total);
  if (!aligned16(workspace))
    return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  // One reading of the split-length override per call; with it, the plan is the
  // batch-invariant one with that minimum split length.
  const int split_tokens = split_tokens_setting().load(std::memory_order_relaxed);
  const bool invariant = (s->flags & GQA_FLAG_BATCH_INVARIANT) || split_tokens > 0;
  const int min_tokens = split_tokens > 0 ? split_tokens : gqa::kMinSplitTokens;
  const int kv = kivi ? 2 : fp8 ? 1 : 0;
  const WavePlan wp = pick_waves(s, row_capacity(rows), kv, fp8 && (positions || append_tail),
                                 invariant);
  const int waves = wp.waves;
  const void* fn = pick_kernel(s->head_dim, s->block_size, row_capacity(rows), kv, waves);
  if (!fn) return fail(GQA_ERR_UNSUPPORTED, "no kernel for this shape");
  const void* tfn = wp.target_waves == waves
                        ? fn
                        : pick_kernel(s->head_dim, s->block_size, row_capacity(rows), kv,
                                      wp.target_waves);
  const int target = target_splits(s, tfn ? tfn : fn, (tfn ? wp.target_waves : waves) * 64,
                                   invariant);
  const int launch_splits =
      split_bound(max_span(s, max_context_len, num_queries), target, min_tokens);
  if ((int64_t)launch_splits * s->num_kv_heads * s->num_seqs > INT32_MAX)
    return fail(GQA_ERR_UNSUPPORTED, "grid too large");
  // Ragged batches: share each KV head's slots out by sequence length (one
  // lane per sequence, so up to 64 sequences) instead of giving every sequence
  // the same number of splits.
  const bool proportional = !invariant && launch_splits >= 2 &&
                            s->num_seqs >= 2 && s->num_seqs <= 64;

  char* ws = static_cast<char*>(workspace);
  gqa::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  // Written only by a fused fp8 append, whose entry points take them non-const.
  p.k_scale = const_cast<float*>(k_scale);
  p.v_scale = const_cast<float*>(v_scale);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.positions = positions;
  p.append_tail = append_tail ? 1 : 0;
  p.out = out;
  p.out_lse = out_lse;
  p.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
  p.ws_lse = reinterpret_cast<float*>(ws + wl.lse_off);
  p.counters = reinterpret_cast<uint32_t*>(ws);
  p.status = reinterpret_cast<uint32_t*>(ws + GQA_WORKSPACE_STATUS_OFFSET);
  p.num_q_heads = s->num_q_heads;
  p.num_kv_heads = s->num_kv_heads;
  p.group = G;
  p.group_shift = __builtin_ctz((unsigned)G);
  p.rows = rows;
  p.num_blocks = s->num_blocks;
  p.max_splits = ws_splits;
  p.proportional = proportional ? 1 : 0;
  // The split merge of 16 rows or more runs in its own kernel, one wave per (row,
  // KV head, sequence) spread over the GPU, instead of one workgroup per (sequence,
  // KV head) after the last split: 8K with 4 positions 17.7 -> 17.2 us, 32K with
  // 4 positions 92.5 -> 91.0 us.  Lighter merges are faster in the decode launch
  // (8K, 4 rows: 13.2 against 15.2 us with the second kernel).
  const bool defer = launch_splits >= 2 && (defer_merge_override() == 1 ||
                                            (defer_merge_override() == 0 && row_capacity(rows) >= 16));
  p.defer_merge = defer ? 1 : 0;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  // The leading scalar arguments of paged_decode_kernel (preloaded into SGPRs).
  const int32_t* bt_arg = block_tables;
  const int32_t* lens_arg = context_lens;
  int32_t hint_arg = max_context_len;
  int32_t max_blocks_arg = s->max_blocks_per_seq;
  int32_t window_arg = s->sliding_window;
  // bits 0-7 split target, 8 proportional sharing, 16-23 query positions; the
  // split-length override T as T / 32 in bits 9-15 (low) and 24-31 (high), 0 if none
  const uint32_t split32 = split_tokens > 0 ? (uint32_t)split_tokens / gqa::kChunkTokens : 0u;
  int32_t plan_arg = (int32_t)((uint32_t)target | (proportional ? 1u << 8 : 0u) |
                               ((split32 & 0x7fu) << 9) | ((uint32_t)num_queries << 16) |
                               ((split32 >> 7) << 24));
  if (clear_counters) {
    // A shared workspace (the static scratch): zero its arrival counters and status
    // word with a fill kernel on the same stream, after every argument was checked.
    uint32_t* words = p.counters;
    size_t n = wl.cnt_words;
    void* zargs[] = {&words, &n};
    const unsigned zb = (unsigned)((n + 255) / 256 > 1024 ? 1024 : (n + 255) / 256);
    const hipError_t ze = hipLaunchKernel(reinterpret_cast<const void*>(&gqa::zero_words_kernel),
                                          dim3(zb), dim3(256), zargs, 0, stream);
    if (ze != hipSuccess)
      return fail(GQA_ERR_HIP, "clearing the workspace counters failed: %s", hipGetErrorString(ze));
  }
  void* args[] = {&bt_arg, &lens_arg, &hint_arg, &max_blocks_arg, &window_arg, &plan_arg, &p};
  const hipError_t e = hipLaunchKernel(fn, dim3(launch_splits, s->num_kv_heads, s->num_seqs),
                                       dim3(waves * 64), args, 0, stream);
  if (e != hipSuccess)
    return fail(GQA_ERR_HIP, "paged_decode launch failed: %s", hipGetErrorString(e));
  if (defer) {
    const float* mo = p.ws_o;
    const float* ml = p.ws_lse;
    const uint32_t* mc = p.counters;
    int32_t hkv = s->num_kv_heads, mcap = row_capacity(rows), msplits = ws_splits, nq = num_queries;
    int32_t scap = launch_splits;                  // splits loaded with the count
    int32_t hq = s->num_q_heads, g = G, gshift = p.group_shift;
    float* mout = out;
    float* mlse = out_lse;
    void* margs[] = {&mo, &ml, &mc, &hkv, &mcap, &msplits, &scap, &nq, &hq, &g, &gshift, &mout, &mlse};
    const void* mfn = s->head_dim == 64 ? reinterpret_cast<const void*>(&gqa::merge_splits_kernel<64>)
                                        : reinterpret_cast<const void*>(&gqa::merge_splits_kernel<128>);
    const hipError_t me = hipLaunchKernel(mfn, dim3(rows, s->num_kv_heads, s->num_seqs), dim3(64),
                                          margs, 0, stream);
    if (me != hipSuccess)
      return fail(GQA_ERR_HIP, "split merge launch failed: %s", hipGetErrorString(me));
  }
  return ok();
}

gqa_status gqa_paged_decode_attention(const gqa_paged_shape* s, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t max_context_len, float softmax_scale, float* out,
                                      float* out_lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  return decode_impl(s, 1, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), k_scale,
                     v_scale, nullptr, nullptr, nullptr, block_tables, context_lens,
                     max_context_len, softmax_scale, out, out_lse, workspace, workspace_bytes,
                     stream);
}

gqa_status gqa_paged_decode_multi_query(const gqa_paged_shape* s, int32_t num_queries,
                                        const void* q, const void* k_cache, const void* v_cache,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        int32_t max_context_len, float softmax_scale, float* out,
                                        float* out_lse, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  return decode_impl(s, num_queries, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                     k_scale, v_scale, nullptr, nullptr, nullptr, block_tables, context_lens,
                     max_context_len, softmax_scale, out, out_lse, workspace, workspace_bytes,
                     stream);
}

gqa_status gqa_paged_decode_multi_query_append(
    const gqa_paged_shape* s, int32_t num_queries, const void* q, const void* k_new,
    const void* v_new, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
    const int32_t* block_tables, const int32_t* context_lens, int32_t max_context_len,
    float softmax_scale, float* out, float* out_lse, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  return decode_impl(s, num_queries, q, k_cache, v_cache, k_scale, v_scale, k_new, v_new,
                     nullptr, block_tables, context_lens, max_context_len, softmax_scale, out,
                     out_lse, workspace, workspace_bytes, stream, true);
}

gqa_status gqa_paged_decode_append_attention(
    const gqa_paged_shape* s, const void* q, const void* k_new, const void* v_new,
    const int32_t* positions, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
    const int32_t* block_tables, const int32_t* context_lens, int32_t max_context_len,
    float softmax_scale, float* out, float* out_lse, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  if (s && s->num_seqs > 0 && !positions)
    return fail(GQA_ERR_INVALID_ARG, "append: NULL positions");
  return decode_impl(s, 1, q, k_cache, v_cache, k_scale, v_scale, k_new, v_new, positions,
                     block_tables, context_lens, max_context_len, softmax_scale, out, out_lse,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

// The workspace of gqa_paged_decode_attention_noalloc: one array per device, in
// the library's own device memory (allocated when the code object loads, held
// until the process ends).  In host code `scratch` names a host-side stand-in,
// not a device address: host code uses the address hipGetSymbolAddress gives
// for the current device, never the name.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per device.
gqa_status scratch_address(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "noalloc: hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GQA_ERR_HIP, "noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    it = addr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_paged_decode_attention_noalloc(const gqa_paged_shape* s, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const float* k_scale, const float* v_scale,
                                              const int32_t* block_tables,
                                              const int32_t* context_lens,
                                              int32_t max_context_len, float softmax_scale,
                                              float* out, float* out_lse, hipStream_t stream) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (max_context_len < 0)
    return fail(GQA_ERR_INVALID_ARG, "max_context_len %d < 0", max_context_len);
  if (s->num_seqs == 0) return ok();
  const size_t need = gqa_paged_decode_workspace_size(s, max_context_len);
  if (need > (size_t)GQA_NOALLOC_SCRATCH_BYTES)
    return fail(GQA_ERR_WORKSPACE, "noalloc: this call needs %zu bytes of workspace, more than "
                "the %zu-byte static scratch (use gqa_paged_decode_attention with a workspace)",
                need, (size_t)GQA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != GQA_OK) return st;
  // Every call on a device shares its scratch, which keeps the last call's
  // contents: decode_impl zeroes the counters and status word first.
  return decode_impl(s, 1, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), k_scale,
                     v_scale, nullptr, nullptr, nullptr, block_tables, context_lens,
                     max_context_len, softmax_scale, out, out_lse, ws,
                     (size_t)GQA_NOALLOC_SCRATCH_BYTES, stream, false, true);
}

gqa_status gqa_paged_decode_workspace_init(const gqa_paged_shape* s, int32_t max_context_len,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (max_context_len < 0)
    return fail(GQA_ERR_INVALID_ARG, "max_context_len %d < 0", max_context_len);
  const WorkspaceLayout wl = workspace_layout(s, max_splits_for(max_context_len), 1);
  if (!workspace || workspace_bytes < wl.cnt_words * sizeof(uint32_t))
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                wl.cnt_words * sizeof(uint32_t));
  if (wl.cnt_words == 0) return ok();
  uint32_t* cnt = static_cast<uint32_t*>(workspace);
  size_t n = wl.cnt_words;
  struct {
    uint32_t* w;
    size_t n;
  } args{cnt, n};
  void* argv[] = {&args.w, &args.n};
  const unsigned blocks = (unsigned)((n + 255) / 256 > 1024 ? 1024 : (n + 255) / 256);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&gqa::zero_words_kernel),
                                 dim3(blocks), dim3(256), argv, 0, stream);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "workspace init failed: %s", hipGetErrorString(e));
  return ok();
}

gqa_status gqa_workspace_read_status(const void* workspace, size_t workspace_bytes, int32_t clear,
                                     uint32_t* status, hipStream_t stream) {
  if (!workspace || !status)
    return fail(GQA_ERR_INVALID_ARG, "read_status: NULL workspace or status");
  if (workspace_bytes < GQA_WORKSPACE_STATUS_OFFSET + sizeof(uint32_t))
    return fail(GQA_ERR_WORKSPACE, "read_status: workspace of %zu bytes holds no status word",
                workspace_bytes);
  uint32_t* word = reinterpret_cast<uint32_t*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                               GQA_WORKSPACE_STATUS_OFFSET);
  uint32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, word, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "read_status: %s", hipGetErrorString(e));
  *status = host;
  if (clear && host != 0) {
    size_t n = 1;
    void* argv[] = {&word, &n};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&gqa::zero_words_kernel), dim3(1), dim3(64),
                        argv, 0, stream);
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "read_status: clear failed: %s",
                                     hipGetErrorString(e));
  }
  return ok();
}

gqa_status gqa_kv_copy_blocks(const gqa_paged_shape* s, void* k_cache, void* v_cache,
                              float* k_scale, float* v_scale, const int32_t* src_blocks,
                              const int32_t* dst_blocks, int32_t num_pairs, hipStream_t stream) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (num_pairs < 0 || num_pairs > INT32_MAX / 2)
    return fail(GQA_ERR_INVALID_ARG, "num_pairs %d out of range", num_pairs);
  const bool fp8 = s->kv_dtype != GQA_KV_BF16;
  const bool kivi = s->kv_dtype == GQA_KV_FP8_E4M3_KIVI;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr))
    return fail(GQA_ERR_INVALID_ARG, "k_scale/v_scale are required for fp8 pools and must be "
                "NULL for bf16");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks)
    return fail(GQA_ERR_INVALID_ARG, "copy_blocks: NULL device pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(GQA_ERR_INVALID_ARG, "copy_blocks: pools must be 16-byte aligned");
  gqa::CopyBlocksParams p;
  p.k_cache = static_cast<char*>(k_cache);
  p.v_cache = static_cast<char*>(v_cache);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.src = src_blocks;
  p.dst = dst_blocks;
  p.num_blocks = s->num_blocks;
  p.k_scales = s->num_kv_heads * (kivi ? s->head_dim : 1);
  p.v_scales = s->num_kv_heads * (kivi ? s->block_size : 1);
  p.block_bytes = (int64_t)s->num_kv_heads * s->block_size * s->head_dim * (fp8 ? 1 : 2);
  const int64_t slices = (p.block_bytes + gqa::kCopySliceBytes - 1) / gqa::kCopySliceBytes;
  // One workgroup of kCopyThreads per work item, and a dispatch counts its grid in
  // threads with 32 bits: at most UINT32_MAX / kCopyThreads (2^24 - 1) work items.
  const int64_t max_items = (int64_t)UINT32_MAX / gqa::kCopyThreads;
  if ((int64_t)num_pairs * slices > max_items)
    return fail(GQA_ERR_INVALID_ARG, "copy_blocks: %d pairs of %lld-byte blocks exceed one "
                "launch (%lld 4 KiB slices, at most %lld)", num_pairs, (long long)p.block_bytes,
                (long long)num_pairs * slices, (long long)max_items);
  p.slices = (int32_t)slices;
  p.work_items = (uint32_t)(num_pairs * slices);
  st = launch(reinterpret_cast<const void*>(&gqa::kv_copy_blocks_kernel), dim3(p.work_items),
              dim3(gqa::kCopyThreads), &p, "kv_copy_blocks", stream);
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_kv_gather(const gqa_paged_shape* s, const void* cache, const int32_t* block_tables,
                         int32_t seq, int32_t num_tokens, void* out, hipStream_t stream) {
  gqa_status st = check_shape(s);
  if (st != GQA_OK) return st;
  if (seq < 0 || seq >= s->num_seqs)
    return fail(GQA_ERR_INVALID_ARG, "seq %d out of range [0, %d)", seq, s->num_seqs);
  if (num_tokens < 0 || (int64_t)num_tokens > (int64_t)s->max_blocks_per_seq * s->block_size)
    return fail(GQA_ERR_INVALID_ARG, "num_tokens %d out of range", num_tokens);
  if (num_tokens == 0) return ok();
  if (!cache || !block_tables || !out) return fail(GQA_ERR_INVALID_ARG, "gather: NULL pointer");
  if (!aligned16(cache) || !aligned16(out))
    return fail(GQA_ERR_INVALID_ARG, "gather: pointers must be 16-byte aligned");
  gqa::GatherParams p;
  p.cache = static_cast<const char*>(cache);
  p.block_table = block_tables + (size_t)seq * s->max_blocks_per_seq;
  p.out = static_cast<char*>(out);
  p.num_kv_heads = s->num_kv_heads;
  p.block_size = s->block_size;
  p.num_blocks = s->num_blocks;
  p.num_tokens = num_tokens;
  p.row_bytes = s->head_dim * (s->kv_dtype != GQA_KV_BF16 ? 1 : 2);
  st = launch(reinterpret_cast<const void*>(&gqa::kv_gather_kernel),
              dim3((num_tokens + 63) / 64, s->num_kv_heads), dim3(256), &p, "kv_gather", stream);
  return st == GQA_OK ? ok() : st;
}

}  // extern "C"
