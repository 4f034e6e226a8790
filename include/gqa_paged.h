/*
 * gqa_paged.h — C ABI of the MI355X (gfx950) paged GQA decode-attention library.
 *
 * The library computes decode attention over a paged KV cache with grouped
 * query heads (one query position per sequence, or a few consecutive ones, as
 * when verifying speculative tokens), and the KV append that commits new
 * tokens before it.
 *
 * What the operations are, and where the pages state them:
 *  - KV cache and append: each step commits the pending token's K/V, then its
 *    query attends over the cache including itself.  *LLM Inference Systems
 *    Engineering* (jasonzhang109) §2.1.3; *The Mathematics of Transformer
 *    Inference* (hs-black) §1.
 *  - Paging: fixed-size physical blocks in one shared pool, a per-sequence block
 *    table from logical to physical block; a sequence's blocks need not be
 *    adjacent; the attention kernel reads K/V through the table and only reads
 *    each sequence's valid tokens.  *Module 10: Inference and Deployment Serving*
 *    (wrwei.github.io), "Mapping logical positions to physical blocks";
 *    *The Mathematics of Transformer Inference* §9 (PagedAttention).
 *  - Decode attention with grouped queries: query head h reads KV head
 *    floor(h / G), G = H_q / H_kv; scores are softmax_scale * <q, k>, the output
 *    is the softmax-weighted sum of values.  *The Mathematics of Transformer
 *    Inference* §4-5; *Module 10*, Lab 2 (KV heads repeated over consecutive
 *    query heads).
 *  - FP8 KV: E4M3 in the finite-only convention (max 448), dequantised inside the
 *    kernel with a scale.  *Module 10*, number-format table; *The Mathematics of
 *    Transformer Inference* §11.
 *  - Sliding window: a local-attention layer keeps only a bounded recent context
 *    (the w most recent tokens; Mistral 7B uses w = 4096).  *Module 10*,
 *    "Parameter count alone does not determine cache size"; *The Mathematics of
 *    Transformer Inference* §5.  With a window, table entries of blocks that lie
 *    wholly before every query's window are never read (they may be released).
 *  - Several query positions per sequence: speculative decoding verifies k
 *    drafted tokens with one target pass over the committed prefix plus those
 *    positions, each attending causally.  *LLM Inference Systems Engineering*
 *    §2.1.3 (the verification interface); *The Mathematics of Transformer
 *    Inference* §10.
 *
 * Conventions shared by all calls
 *  - All pointers except `shape` are DEVICE pointers on the current HIP device,
 *    owned by the caller.  The library allocates nothing and keeps no device
 *    state between calls.  Every call is asynchronous on `stream` (0 = null
 *    stream) and only enqueues work; results are ready when the stream is.
 *  - bf16 values are raw bfloat16 bit patterns (uint16); fp8 values are OCP
 *    E4M3 codes (uint8; 0x7F/0xFF are NaN, no infinity).
 *  - KV pool layout: k_cache, v_cache are [num_blocks][num_kv_heads][block_size][head_dim]
 *    (row-major), so one (block, KV head) tile is contiguous.  Token t of sequence b
 *    lives in physical block block_tables[b * max_blocks_per_seq + t / block_size]
 *    at slot t % block_size.  Table entries at or beyond ceil(ctx_b / block_size)
 *    are never read.
 *  - Supported shapes: head_dim in {64, 128}; block_size in {16, 32};
 *    num_q_heads % num_kv_heads == 0 with G = num_q_heads / num_kv_heads in
 *    {1, 2, 4, 8, 16, 32}, and G * (query positions) <= 32 rows per KV head
 *    (<= 8 for KIVI pools); kv_dtype BF16 or FP8_E4M3.  Anything else returns
 *    GQA_ERR_UNSUPPORTED.  Device pointers must be 16-byte aligned.
 *  - Errors: a call validates its host-side arguments and returns a status; it
 *    never aborts.  gqa_last_error() gives a message for the last non-OK status
 *    on the calling thread.  Device-resident values (block ids, positions,
 *    context lengths) are checked inside the kernels: a sequence whose context
 *    length or attended block ids are out of range gets NaN in every output
 *    element and lse of its heads (nothing outside the buffers is read), and an
 *    append whose position or block id is out of range writes nothing.  The
 *    attention calls also record each such fault as a GQA_STATUS_* bit in the
 *    workspace's status word, which gqa_workspace_read_status returns, so the
 *    host can tell a corrupted table or length from NaN data.
 *  - Tuning overrides, read once per process from the environment: GQA_WAVES
 *    (4 or 8 waves per workgroup) and GQA_SPLIT_ROUNDS (r >= 1: size the context
 *    split target for r rounds of the GPU's resident workgroups instead of one).
 *    Unset, the library chooses; neither applies under GQA_FLAG_BATCH_INVARIANT.
 *    Like any split plan they change results in the last bits only.
 *    GQA_DEFER_MERGE = 1 merges the context splits in a second kernel launch (on
 *    the same stream), 2 in the attention launch itself; unset, calls with 16 or
 *    more query rows per KV head use the second launch.  The merge arithmetic is
 *    the same either way; its summation order differs.
 *  - Split-length override: GQA_SPLIT_TOKENS (read once per process, or set at
 *    run time with gqa_set_split_tokens) = T, a multiple of 32 in [128, 2^19].
 *    When set, every attention call splits each sequence by its own length
 *    into about one split per T tokens (at most 64; gqa_decode_num_splits), as under
 *    GQA_FLAG_BATCH_INVARIANT with T in place of 128: results stay
 *    batch-invariant, and T trades that mode's split count for its cost.
 */
#ifndef GQA_PAGED_H
#define GQA_PAGED_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, misaligned pointer  */
  GQA_ERR_UNSUPPORTED = 2,   /* valid but unsupported head_dim/block_size/G/dtype */
  GQA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required        */
  GQA_ERR_HIP = 4            /* a HIP launch failed; see gqa_last_error()         */
} gqa_status;

/* Stored K/V element type and, for fp8, the layout of the fp32 scales
 * (value = decode(code) * scale):
 *   GQA_KV_FP8_E4M3       k_scale, v_scale [num_blocks][H_kv]: one per (block, KV head)
 *   GQA_KV_FP8_E4M3_KIVI  k_scale [num_blocks][H_kv][head_dim]: one per channel of each
 *                         (block, KV head); v_scale [num_blocks][H_kv][block_size]: one
 *                         per token (slot) -- keys per channel and values per token, as
 *                         KIVI quantises them (*Module 10*, "Quantize the cache"; *The
 *                         Mathematics of Transformer Inference* §11). */
typedef enum gqa_kv_dtype {
  GQA_KV_BF16 = 0,
  GQA_KV_FP8_E4M3 = 1,
  GQA_KV_FP8_E4M3_KIVI = 2
} gqa_kv_dtype;

/* Shape flags. */
enum {
  /* Split every sequence's context by its own length only (the split plan of
   * gqa_decode_num_splits), so a sequence's attention result is bit-identical
   * whatever else is in the batch.  Without it the split count also follows
   * the batch size (more, shorter splits when the batch is small), which is
   * faster but makes results depend on the batch size in the last bits; they
   * never depend on the order of the sequences. */
  GQA_FLAG_BATCH_INVARIANT = 1
};

/* Device status bits.  The attention calls (all of which take a workspace) OR
 * these into the 32-bit word at byte GQA_WORKSPACE_STATUS_OFFSET of their
 * workspace when they meet a bad device-resident input.  The bits are sticky:
 * no call clears them; gqa_workspace_read_status (clear = 1) or
 * gqa_paged_decode_workspace_init does.  The table and length contract they
 * check is that of *Module 10*, "Mapping logical positions to physical
 * blocks", and *The Mathematics of Transformer Inference* §9: every logical
 * block a sequence attends maps to a physical block of the pool. */
enum {
  GQA_STATUS_BAD_CONTEXT_LEN = 1,   /* context_lens[b] < 0, beyond max_blocks_per_seq *
                                       block_size, or 0 < context_lens[b] < num_queries  */
  GQA_STATUS_CONTEXT_OVER_HINT = 2, /* context_lens[b] > max_context_len (the launch hint) */
  GQA_STATUS_BAD_BLOCK_ID = 4,      /* an attended table entry outside [0, num_blocks)    */
  GQA_STATUS_BAD_APPEND = 8         /* a fused append's position is past the table, or its
                                       table entry is not a block of the pool            */
};
#define GQA_WORKSPACE_STATUS_OFFSET 4

/* Host-side description of one paged KV cache and one batch of sequences. */
typedef struct gqa_paged_shape {
  int32_t num_seqs;            /* B: sequences in the batch (0 is a no-op)           */
  int32_t num_q_heads;         /* H_q                                                 */
  int32_t num_kv_heads;        /* H_kv; H_q % H_kv == 0                               */
  int32_t head_dim;            /* d_h                                                 */
  int32_t block_size;          /* BS tokens per physical block                        */
  int32_t num_blocks;          /* physical blocks in each pool                        */
  int32_t max_blocks_per_seq;  /* row length of block_tables                          */
  int32_t kv_dtype;            /* gqa_kv_dtype                                        */
  int32_t flags;               /* GQA_FLAG_* bits (0 = default)                      */
  int32_t sliding_window;      /* w > 0: each query attends to its w most recent     */
                               /* tokens, itself included; 0: the whole context      */
} gqa_paged_shape;

/*
 * gqa_kv_append — commit one new token per sequence into the paged pools.
 *   k_new, v_new  [B][H_kv][d_h] bf16       the token's key and value rows
 *   k_cache, v_cache  pools (layout above), modified in place
 *   block_tables  [B][max_blocks_per_seq] int32
 *   positions     [B] int32: logical slot to write (usually ctx_b - 1, the new
 *                 token's index); a negative position skips that sequence
 * Writes k_cache[blk][h][pos % BS][:] = k_new[b][h][:] (same for V) with
 * blk = block_tables[b][pos / BS]; a bit-exact copy.  context_lens is not
 * touched: the caller passes the grown length to the attention call.
 * bf16 pools only (GQA_ERR_UNSUPPORTED for fp8): fp8 pools are appended to,
 * quantising, with gqa_kv_append_fp8.
 */
gqa_status gqa_kv_append(const gqa_paged_shape* shape,
                         const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache,
                         const int32_t* block_tables, const int32_t* positions,
                         hipStream_t stream);

/*
 * gqa_kv_append_tokens — commit num_tokens new tokens per sequence (for
 * example a pending token and its drafts before verification).
 *   num_tokens    T in [0, 65535]
 *   k_new, v_new  [B][T][H_kv][d_h] bf16 rows
 *   positions     [B][T] int32 logical slots; a position outside
 *                 [0, max_blocks_per_seq * block_size) skips that token
 *   other arguments as gqa_kv_append, which is the T = 1 case.  Tokens are
 *   copied independently (bit-exact); two tokens given the same slot leave
 *   either one there.  bf16 pools only (fp8: gqa_kv_append_fp8).
 */
gqa_status gqa_kv_append_tokens(const gqa_paged_shape* shape, int32_t num_tokens,
                                const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache,
                                const int32_t* block_tables, const int32_t* positions,
                                hipStream_t stream);

/*
 * gqa_decode_num_splits — the batch-invariant context split plan (host
 * function, no GPU): how many partial attentions a sequence of `context_len`
 * attended tokens is cut into under GQA_FLAG_BATCH_INVARIANT, with the current
 * split-length override T if one is set (else T = 128):
 * n = min(64, ceil(context_len / T)) splits of ceil(context_len / n) tokens
 * rounded up to a multiple of 32, the last one shorter.  0 for
 * context_len <= 0.  No plan uses more than min(64, ceil(context_len / 128)).
 * The split-K decomposition with a log-sum-exp merge of the pieces is that of
 * *The Mathematics of Transformer Inference* §8 (sequence shards merged by
 * their log-sum-exp), applied to context ranges on one GPU.
 */
int32_t gqa_decode_num_splits(int32_t context_len);

/*
 * gqa_set_split_tokens — set (tokens = T, a multiple of 32 in [128, 2^19]) or
 * clear (tokens = 0) the process-wide split-length override that
 * GQA_SPLIT_TOKENS sets at start-up.  Calls made after it returns use the new
 * value; a call already being launched on another thread may use either.
 * Returns GQA_ERR_INVALID_ARG (and keeps the old value) for any other value.
 * Launches captured in a HIP graph keep the plan they were captured with.
 * gqa_split_tokens returns the current value (0 when none is set).
 */
gqa_status gqa_set_split_tokens(int32_t tokens);
int32_t gqa_split_tokens(void);

/*
 * gqa_paged_decode_workspace_size — bytes of device workspace that
 * gqa_paged_decode_attention needs for this shape when no sequence is longer
 * than max_context_len.  Returns 0 for invalid or unsupported arguments.
 */
size_t gqa_paged_decode_workspace_size(const gqa_paged_shape* shape, int32_t max_context_len);

/*
 * gqa_paged_decode_attention — one decode step of attention for B sequences.
 *   q             [B][H_q][d_h] bf16
 *   k_cache, v_cache  pools (layout above); bf16 or fp8 codes
 *   k_scale, v_scale  fp32 dequantisation scales for fp8 pools (value =
 *                 decode(code) * scale): [num_blocks][H_kv], or for
 *                 GQA_KV_FP8_E4M3_KIVI k_scale [num_blocks][H_kv][d_h] and
 *                 v_scale [num_blocks][H_kv][block_size]; must be NULL for bf16
 *   block_tables  [B][max_blocks_per_seq] int32
 *   context_lens  [B] int32: tokens each sequence attends, including a token
 *                 just appended; 0 gives out = 0, lse = -inf
 *   max_context_len  host bound on every context_lens[b]; sizes the launch.
 *                 A sequence longer than this gets NaN output.
 *   softmax_scale score multiplier (usually 1/sqrt(d_h))
 *   out           [B][H_q][d_h] fp32 (written)
 *   out_lse       [B][H_q] fp32 natural-log log-sum-exp of the scores, or NULL
 *   workspace     device scratch of at least
 *                 gqa_paged_decode_workspace_size(shape, max_context_len) bytes,
 *                 16-byte aligned.  It starts with one arrival counter (u32) per
 *                 (sequence, KV head), 256 bytes apart, followed by the partial
 *                 results of the context splits; the word at byte
 *                 GQA_WORKSPACE_STATUS_OFFSET (in the first counter's 256 bytes) is
 *                 the status word.  The first B*H_kv*64 words
 *                 (B*H_kv*256 bytes) must be zero before the first
 *                 call (gqa_paged_decode_workspace_init, or any zero fill); every
 *                 call leaves each arrival counter (the first word of its 256
 *                 bytes) zero again, so a workspace prepared once
 *                 serves any later call with no more (sequence, KV head) pairs (the
 *                 status word keeps its bits until cleared).  One
 *                 workspace serves one call at a time: calls sharing it must be
 *                 ordered on one stream.
 * Inputs are read only.  One kernel runs on `stream`: each workgroup attends
 * over one context split of one (sequence, KV head); the last workgroup of a
 * (sequence, KV head) to finish merges the splits by log-sum-exp.  With 16 or
 * more query rows per KV head (or GQA_DEFER_MERGE=1) the splits merge in a
 * second kernel on the same stream instead.
 */
gqa_status gqa_paged_decode_attention(const gqa_paged_shape* shape,
                                      const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_tables,
                                      const int32_t* context_lens,
                                      int32_t max_context_len,
                                      float softmax_scale,
                                      float* out, float* out_lse,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * gqa_paged_multi_query_workspace_size — workspace bytes for
 * gqa_paged_decode_multi_query with num_queries positions per sequence (equal
 * to gqa_paged_decode_workspace_size when num_queries is 1).  0 for invalid
 * arguments.
 */
size_t gqa_paged_multi_query_workspace_size(const gqa_paged_shape* shape, int32_t num_queries,
                                            int32_t max_context_len);

/*
 * gqa_paged_decode_multi_query — attention for Q consecutive query positions
 * per sequence over the paged cache, as in the verification pass of
 * speculative decoding or a short chunk of prefill onto a cache.
 *   num_queries   Q >= 1, with G * Q <= 32 (<= 8 for GQA_KV_FP8_E4M3_KIVI pools)
 *                 (else GQA_ERR_UNSUPPORTED)
 *   q             [B][Q][H_q][d_h] bf16; query i of sequence b sits at position
 *                 context_lens[b] - Q + i, so the Q new tokens must already be
 *                 in the cache (gqa_kv_append_tokens)
 *   context_lens  [B] int32 tokens in the cache including the Q new ones.
 *                 Query i attends to tokens 0 .. context_lens[b] - Q + i
 *                 (causal among the new positions).  0 gives out = 0 and
 *                 lse = -inf; 0 < context_lens[b] < Q gives NaN.
 *   out           [B][Q][H_q][d_h] fp32; out_lse [B][Q][H_q] fp32 or NULL
 *   workspace     at least gqa_paged_multi_query_workspace_size(shape,
 *                 num_queries, max_context_len) bytes, counters as described
 *                 for gqa_paged_decode_attention
 *   other arguments as gqa_paged_decode_attention, which is the Q = 1 case
 *   (same kernel, same bits).
 */
gqa_status gqa_paged_decode_multi_query(const gqa_paged_shape* shape, int32_t num_queries,
                                        const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* block_tables,
                                        const int32_t* context_lens,
                                        int32_t max_context_len,
                                        float softmax_scale,
                                        float* out, float* out_lse,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/*
 * gqa_paged_decode_multi_query_append — the fused verification step: commit
 * the Q new tokens of every sequence, then attend for all Q positions, in one
 * kernel.
 *   k_new, v_new  [B][Q][H_kv][d_h] bf16: row i goes to position
 *                 context_lens[b] - Q + i (the sequence's last Q tokens)
 *   other arguments as gqa_paged_decode_multi_query (k_cache/v_cache are
 *   written at those Q slots only).  Same results as gqa_kv_append_tokens at
 *   those positions followed by gqa_paged_decode_multi_query.  A sequence with
 *   an invalid length (NaN outputs) appends nothing.
 *   fp8 pools: k_scale/v_scale are required and updated; the rows are
 *   quantised as gqa_kv_append_fp8 with start = context_lens[b] - Q does
 *   (same codes and scales), then attended.  Q <= block_size.
 */
gqa_status gqa_paged_decode_multi_query_append(const gqa_paged_shape* shape,
                                               int32_t num_queries, const void* q,
                                               const void* k_new, const void* v_new,
                                               void* k_cache, void* v_cache,
                                               float* k_scale, float* v_scale,
                                               const int32_t* block_tables,
                                               const int32_t* context_lens,
                                               int32_t max_context_len,
                                               float softmax_scale,
                                               float* out, float* out_lse,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/*
 * gqa_paged_decode_append_attention — one fused decode step ("forward and
 * commit"): write each sequence's new token into the cache, then attend over
 * context_lens[b] tokens that include it, in a single kernel.
 *   k_new, v_new  [B][H_kv][d_h] bf16 new rows; positions [B] int32 slot of the
 *                 new token (normally context_lens[b] - 1; negative = no append)
 *   other arguments as gqa_paged_decode_attention (k_cache/v_cache are written
 *   at the appended slots only).  Same results as gqa_kv_append followed by
 *   gqa_paged_decode_attention.  fp8 pools: k_scale/v_scale (NULL for bf16)
 *   are required and updated; the row is quantised as gqa_kv_append_fp8 with
 *   start = positions[b] does (same codes and scales), then attended.
 * Cites: *LLM Inference Systems Engineering* §2.1.3 (each step commits the
 * pending token's K/V, then attends over the cache that includes it).
 */
gqa_status gqa_paged_decode_append_attention(const gqa_paged_shape* shape,
                                             const void* q,
                                             const void* k_new, const void* v_new,
                                             const int32_t* positions,
                                             void* k_cache, void* v_cache,
                                             float* k_scale, float* v_scale,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens,
                                             int32_t max_context_len,
                                             float softmax_scale,
                                             float* out, float* out_lse,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/*
 * gqa_paged_decode_workspace_init — zero the arrival counters (the first
 * B*H_kv*64 words, the status word among them) of a workspace; workspace_bytes
 * must cover them.  Enqueued on
 * `stream` as a small fill kernel (no memset), so it may be captured in a HIP
 * graph.  max_context_len is validated but does not change what is zeroed.
 */
gqa_status gqa_paged_decode_workspace_init(const gqa_paged_shape* shape, int32_t max_context_len,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/*
 * gqa_paged_decode_attention_noalloc — gqa_paged_decode_attention without a
 * caller-supplied workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments without workspace/workspace_bytes, same kernel
 * and the same results bit for bit.  Its workspace is a static array of
 * GQA_NOALLOC_SCRATCH_BYTES in the library's device memory, one per device,
 * held until the process ends; the call allocates nothing.  A call whose
 * workspace (gqa_paged_decode_workspace_size) exceeds that size returns
 * GQA_ERR_WORKSPACE.  Each call first zeroes the scratch's arrival counters and
 * status word with a small fill kernel on `stream`, then launches the decode
 * kernel: two kernels, both capturable in a HIP graph.  All calls on one device
 * share the array, so calls that overlap in time on one device (on different
 * streams, or from different threads without ordering) race and give wrong
 * results: order them on one stream.
 */
#define GQA_NOALLOC_SCRATCH_BYTES (32u << 20)
gqa_status gqa_paged_decode_attention_noalloc(const gqa_paged_shape* shape,
                                              const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const float* k_scale, const float* v_scale,
                                              const int32_t* block_tables,
                                              const int32_t* context_lens,
                                              int32_t max_context_len,
                                              float softmax_scale,
                                              float* out, float* out_lse,
                                              hipStream_t stream);

/*
 * gqa_workspace_read_status — the GQA_STATUS_* bits that the attention calls
 * enqueued so far on `stream` have recorded in this workspace (0: none met a bad
 * device-resident input).  Blocking: copies the word to the host after the
 * stream's earlier work and waits for the stream.  clear != 0 then enqueues a
 * zero fill of the word on `stream` (a small kernel, no memset).
 *   workspace, workspace_bytes  a workspace of the attention calls (device)
 *   status        host pointer receiving the bits
 * Returns GQA_ERR_INVALID_ARG for NULL pointers, GQA_ERR_WORKSPACE when
 * workspace_bytes does not reach the word, GQA_ERR_HIP when the copy fails.
 * Cites: *Module 10*, "Mapping logical positions to physical blocks"; *The
 * Mathematics of Transformer Inference* §9 (the table contract checked).
 */
gqa_status gqa_workspace_read_status(const void* workspace, size_t workspace_bytes,
                                     int32_t clear, uint32_t* status, hipStream_t stream);

/*
 * gqa_kv_append_fp8 — append num_tokens (T) new tokens per sequence to an fp8
 * (E4M3) pool, quantising them with one fp32 scale per (block, KV head), or
 * with the KIVI layout (per-channel key scales, per-token value scales).
 *   k_new, v_new  [num_seqs][T][H_kv][head_dim] bf16 rows, finite (as are the
 *                 codes already in a block the call appends to)
 *   k_cache, v_cache  [num_blocks][H_kv][block_size][head_dim] E4M3 codes, and
 *   k_scale, v_scale  fp32 scales in the pool's layout (see gqa_kv_dtype;
 *                 value = decode(code) * scale), modified in place at the
 *                 blocks written
 *   block_tables  [num_seqs][max_blocks_per_seq] int32
 *   start_positions [num_seqs] int32: sequence b writes positions start[b] ..
 *                 start[b] + T - 1 (its current length upward); start < 0: none.
 *                 Positions past the table, or whose table entry is not a block
 *                 of the pool, are skipped.
 * Scale policy, per (block, KV head) tile written, with first = the lowest slot
 * written and t = max|new value| / 448: a block opened by the call (first == 0)
 * takes the smallest power of two >= t; a block holding older tokens keeps its
 * scale when that is >= t, and otherwise takes the smallest power of two >= t
 * and has its older codes re-encoded (exact while they stay normal E4M3).  New
 * values are encoded as round-to-nearest-even of clamp(x / scale, -448, 448).
 * KIVI layout: keys follow this rule channel by channel (t, the scale and the
 * re-encoding per channel of the tile); each value row gets the smallest power
 * of two >= max|row| / 448 when it is written.
 * Precondition: no two sequences write the same block in one call.
 * Cites: *The Mathematics of Transformer Inference* §11 (x ~ s * round(x / s);
 * KV scales per head, per token); *Module 10*, "Quantize the cache" (KIVI:
 * per-channel keys, per-token values) and the E4M3 row of its number-format
 * table (largest value 448).
 */
gqa_status gqa_kv_append_fp8(const gqa_paged_shape* shape, int32_t num_tokens,
                             const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             float* k_scale, float* v_scale, const int32_t* block_tables,
                             const int32_t* start_positions, hipStream_t stream);

/*
 * gqa_kv_copy_blocks — the copy-on-write block copy: for j < num_pairs, block
 * dst_blocks[j] of both pools becomes a bit-exact copy of block src_blocks[j]
 * (every KV head and slot, K and V, and for fp8 pools the per-(block, head)
 * scales).  Used before a sequence writes into a block it shares with others
 * (reference counting and table updates are the caller's).
 *   k_cache, v_cache  pools, modified in place at the destination blocks
 *   k_scale, v_scale  the fp8 pools' scales in their layout (see gqa_kv_dtype),
 *                 copied along; must be NULL for bf16
 *   src_blocks, dst_blocks  [num_pairs] int32 device arrays; a pair with an id
 *                 outside [0, num_blocks), or with src == dst, copies nothing
 *   num_pairs     >= 0; one launch covers num_pairs x ceil(block bytes / 4 KiB)
 *                 work items of 256 threads each, at most 2^24 - 1 of them (the
 *                 dispatch's 32-bit thread count; else GQA_ERR_INVALID_ARG)
 * A source may appear in several pairs (a fork copies one block several times).
 * Performance only: pairs sharing a source are best listed next to each other,
 * as a fork produces them; the copies then read it through one XCD's L2.
 * Precondition: no block is the destination of two pairs or both a source and
 * a destination in one call (the copies run concurrently).
 * Cites: *Module 10*, "Share only state with the same identity"; *Stochastic
 * Parrot* vol. 1 ch. 6 §6.4; *The Mathematics of Transformer Inference* §9.
 */
gqa_status gqa_kv_copy_blocks(const gqa_paged_shape* shape, void* k_cache, void* v_cache,
                              float* k_scale, float* v_scale,
                              const int32_t* src_blocks, const int32_t* dst_blocks,
                              int32_t num_pairs, hipStream_t stream);

/*
 * gqa_kv_gather — copy the first num_tokens cached rows of sequence `seq` out
 * of one pool into a contiguous [H_kv][num_tokens][d_h] array (element width
 * of the pool), in logical order.  A bit-exact indexing check of the paged
 * layout; not on the decode path.
 */
gqa_status gqa_kv_gather(const gqa_paged_shape* shape, const void* cache,
                         const int32_t* block_tables, int32_t seq, int32_t num_tokens,
                         void* out, hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* gqa_last_error(void);

/* Library version string. */
const char* gqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PAGED_H */
