/*
 * pa.h -- paged attention on one AMD Instinct MI355X (gfx950): C ABI.
 *
 * The KV cache is a pool of fixed-size physical blocks.  A sequence's tokens
 * are cut into logical blocks of block_size tokens, and a per-sequence block
 * table maps logical block j to a physical block id anywhere in the pool
 * ("vLLM 基本原理", section PagedAttention, items 1-3).  The pool layout is
 * [num_blocks, num_kv_heads, block_size, head_dim] for K and for V alike
 * (intelliparadigm.com article, section 3.1), so token t of a sequence sits in
 * physical block block_tables[s][t / block_size], row t % block_size.  Only the
 * last block of a sequence may be partly filled ("vLLM 基本原理", on-demand
 * allocation); rows past the sequence length are never read.
 *
 * Attention is the weighted lookup of "vLLM 基本原理" (section "Transformer 和
 * Attention"): out = softmax(scale * q K^T) V over the sequence's cached tokens.
 * Query head h reads kv head h / (num_heads / num_kv_heads).
 *
 * Conventions shared by every entry point
 *  - Ownership: the caller allocates and owns every buffer (device memory),
 *    workspace included.  The library allocates no device memory, keeps no
 *    state between calls and never synchronises.  Outputs must not alias
 *    inputs.
 *  - Asynchrony: every call only enqueues kernels on `stream` (NULL = the
 *    default stream) and returns; results are ready when the stream is.
 *  - Errors: invalid scalar arguments or null pointers return a negative
 *    pa_status before any HIP call is made, and nothing is launched.  A failed
 *    launch returns PA_ERR_LAUNCH.  The contents of device arrays (block ids,
 *    lengths, slots) are the caller's contract; the kernels check each one they
 *    use and, instead of touching memory outside the pools, write NaN into the
 *    affected outputs (attention) or skip the token (scatter).
 *  - Supported: block_size 16; head_dim 64 or 128; dtype fp32 or bf16 for
 *    query, caches and output alike, with fp32 accumulation; num_heads a
 *    multiple of num_kv_heads with num_heads / num_kv_heads <= 16.
 *  - Layouts are dense row-major unless a stride argument says otherwise.
 *    Pool element offsets are 64-bit.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or inconsistent */
  PA_ERR_UNSUPPORTED = -3, /* block_size, head_dim, dtype or group size outside the supported set */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than pa_decode_workspace_bytes() */
  PA_ERR_LAUNCH = -5       /* the HIP runtime refused a kernel launch */
} pa_status;

/*
 * pa_reshape_and_cache -- write each new token's K and V into its cache slot.
 *
 * For token i with slot = slot_mapping[i] >= 0, copies key[i, :, :] into
 * key_cache[slot / block_size, :, slot % block_size, :] and value[i] likewise,
 * bit for bit.  A negative slot is padding and writes nothing; a slot at or
 * past num_blocks * block_size is skipped as well.  Each token's K/V is what
 * the cache keeps so later tokens can attend to it ("vLLM 基本原理", section
 * "什么是 KV Cache").
 *
 *  key, value      [num_tokens, num_kv_heads, head_dim]; heads contiguous inside a
 *                  token, tokens key_stride / value_stride elements apart.
 *  key_cache,
 *  value_cache     [num_blocks, num_kv_heads, block_size, head_dim], updated in place.
 *  slot_mapping    int64 [num_tokens].
 *  Two tokens with the same slot are a caller error (which one lands is undefined).
 */
int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int64_t key_stride,
                         int64_t value_stride, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode_workspace_bytes -- workspace pa_decode needs for split-K.
 *
 * Zero when partition_size == 0 (single pass).  Otherwise room for
 *   o_part   fp32 [num_seqs, num_heads, P, head_dim]
 *   lse_part fp32 [num_seqs, num_heads, P]
 * with P = ceil(max_context_len / partition_size), o_part first, lse_part right
 * after it.  lse is the natural-log log-sum-exp of the partition's scaled scores;
 * o_part is that partition's normalised output.
 */
size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                 int partition_size);

/*
 * pa_decode -- one new query token per sequence attends to its whole cache.
 *
 *  out            [num_seqs, num_heads, head_dim], dtype.
 *  query          [num_seqs, num_heads, head_dim], dtype.
 *  key_cache,
 *  value_cache    [num_blocks, num_kv_heads, block_size, head_dim], dtype.
 *  block_tables   int32 [num_seqs, max_blocks_per_seq]; entries past
 *                 ceil(context_lens[s] / block_size) are never read.
 *  context_lens   int32 [num_seqs]: cached tokens of each sequence, the newest
 *                 included (scatter it first).  0 gives a zero output.
 *  shared_prefix_blocks  optional (NULL = none), int32 [num_seqs]: how many
 *                 leading entries of each sequence's block table name physical
 *                 blocks that other sequences of this call also read -- the
 *                 prompt blocks that forked samples keep in common ("vLLM 基本原理",
 *                 section 内存共享) or a cached prefix (xdnf.cn article, section
 *                 六.3).  A performance hint only: those blocks are read with
 *                 the default cache policy so that sequences reading them at the
 *                 same time hit in L2, the others are streamed past the caches.
 *                 Any value (negative, or past the table) gives the same result.
 *  scale          softmax scale (usually 1/sqrt(head_dim)).
 *  partition_size 0: one pass per sequence writes out directly.  Otherwise a
 *                 multiple of block_size: the context is cut into partitions of
 *                 that many tokens, each handled by its own workgroup (split-K);
 *                 sequences with one partition still write out directly, the
 *                 others write per-partition results to the workspace and
 *                 pa_decode_splitk_reduce() must follow on the same stream.
 *  max_context_len an upper bound on context_lens (sizes the grid and the
 *                 workspace when partition_size > 0).  A sequence whose length
 *                 exceeds it, or exceeds max_blocks_per_seq * block_size, gets NaN.
 *  workspace      device buffer of at least pa_decode_workspace_bytes(); may be
 *                 NULL when partition_size == 0.
 */
int pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* context_lens,
              const int32_t* shared_prefix_blocks, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int64_t num_blocks, int max_context_len, float scale,
              int partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
              hipStream_t stream);

/*
 * pa_decode_splitk_reduce -- merge the partition results pa_decode left in the
 * workspace: with M = max_p lse_p and w_p = exp(lse_p - M),
 * out = sum_p w_p o_p / sum_p w_p.  Sequences with at most one partition are
 * left untouched (pa_decode wrote them).  Arguments must match the pa_decode
 * call that filled the workspace.
 */
int pa_decode_splitk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                            const int32_t* context_lens, int num_seqs, int num_heads,
                            int head_dim, int max_context_len, int partition_size,
                            pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_prefill_chunk -- causal attention for a chunk of new tokens per sequence.
 *
 * Chunked prefill splits one prompt over several rounds (xdnf.cn article,
 * section 六.4); each chunk must see every earlier token of its sequence.
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1
 * (C_s rows); its cache already holds L_s = context_lens[s] tokens, this
 * chunk's K/V included (scatter them first), so query row i sits at position
 * L_s - C_s + i and attends to keys 0 .. L_s - C_s + i.
 *
 *  out, query       [num_query_tokens, num_heads, head_dim], dtype.
 *  query_start_loc  int32 [num_seqs + 1], non-decreasing, last entry <= num_query_tokens.
 *  context_lens     int32 [num_seqs], context_lens[s] >= C_s.
 *  max_query_len    upper bound on C_s (sizes the grid).
 * A sequence whose chunk is longer than max_query_len or than its context, or
 * whose context needs more than max_blocks_per_seq blocks, gets NaN rows.
 */
int pa_prefill_chunk(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* query_start_loc,
                     const int32_t* context_lens, int num_seqs, int num_query_tokens,
                     int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int64_t num_blocks, int max_query_len, float scale,
                     pa_dtype dtype, hipStream_t stream);

/* Human-readable name of a pa_status value (static storage). */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
