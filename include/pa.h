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
 *    workspace included.  The library allocates no device memory and never
 *    synchronises; the kernels' entry points keep no state between calls.
 *    The one stateful object is the block manager (pa_bm_*), host memory the
 *    caller creates and destroys.  Outputs must not alias inputs.
 *  - Asynchrony: every call that takes a `stream` only enqueues kernels or
 *    copies on it (NULL = the default stream) and returns; results are ready
 *    when the stream is.  The block manager's calls are plain host calls.
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

/* Element types.  PA_FP8_E4M3 names FP8 cache pools for the calls that only
 * move whole blocks (pa_copy_blocks, pa_swap_blocks); the FP8 attention calls
 * take uint8_t pools and a pa_dtype for their fp32 / bf16 side. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or inconsistent */
  PA_ERR_UNSUPPORTED = -3, /* block_size, head_dim, dtype or group size outside the supported set */
  PA_ERR_WORKSPACE = -4,   /* workspace missing, smaller than pa_decode_workspace_bytes(), or
                              not 16-byte aligned */
  PA_ERR_LAUNCH = -5,      /* the HIP runtime refused a kernel launch or a copy */
  PA_ERR_NO_BLOCKS = -6,   /* block manager: a pool has too few free blocks; nothing changed */
  PA_ERR_SEQ = -7,         /* block manager: unknown or duplicate sequence id, or the sequence
                              is on the wrong side (swapped out / resident) for the call */
  PA_ERR_BUSY = -8,        /* block manager: the call needs data a pending move has not
                              delivered yet; take and run the moves first.  Nothing changed */
  PA_ERR_NO_MEMORY = -9,   /* block manager: host allocation failed */
  PA_ERR_STATE = -10,      /* block manager: an internal invariant does not hold */
  PA_ERR_SCRATCH = -11     /* pa_decode_no_alloc: the split-K partials would not fit the
                              library's fixed buffer (pa_decode_no_alloc_scratch_bytes()) */
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
 * Split-K is not on the pages: it is how this library spreads one long
 * context over many workgroups, for the long-context grouped-query workload
 * it is measured on (32 sequences of 8k-32k tokens, 32 query over 8 kv heads,
 * context partitions of 512 tokens merged by log-sum-exp).  Each partition's
 * result is exact softmax attention over its own keys, and the merge below
 * recovers attention over all of them ("vLLM 基本原理", section "Transformer
 * 和 Attention": the output is the softmax-weighted mean of V).
 *
 * Zero when partition_size == 0 (single pass).  Otherwise room for
 *   o_part   fp32 [num_seqs, num_heads, P, head_dim]
 *   lse_part fp32 [num_seqs, num_heads, P]
 * with P = ceil(max_context_len / partition_size), o_part first, lse_part right
 * after it.  lse is the natural-log log-sum-exp of the partition's scaled scores;
 * o_part is that partition's normalised output.  After lse_part comes the
 * library's own schedule of the call's work units, 4 * (64 + num_seqs * P)
 * bytes; pa_decode rewrites it on every call and pa_decode_splitk_reduce does
 * not read it.
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
 *  workspace      device buffer of at least pa_decode_workspace_bytes(), 16-byte
 *                 aligned; may be NULL when partition_size == 0.
 */
int pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* context_lens,
              const int32_t* shared_prefix_blocks, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int64_t num_blocks, int max_context_len, float scale,
              int partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
              hipStream_t stream);

/*
 * pa_decode_shared_prefix -- pa_decode for a batch in which groups of
 * sequences share their leading blocks, reading each shared block once per
 * group instead of once per sequence.
 *
 * Samples of one prompt keep the prompt's physical blocks in common ("vLLM
 * 基本原理", section 内存共享), and so do requests that hit one cached prefix
 * (xdnf.cn article, section 六.3).  Decode is bound by the bytes it streams
 * (xdnf.cn article, section 六.5), so here a split-K partition made only of
 * such blocks is streamed once and scored against the queries of a window of
 * sharers (see below for its size); each sharer
 * gets the same per-partition partial its own workgroup would have produced,
 * and pa_decode_splitk_reduce() merges them as usual.  Every argument of
 * pa_decode keeps its meaning, with these differences:
 *
 *  shared_prefix_blocks  required: int32 [num_seqs], leading table entries of
 *                 each sequence that other sequences of its group also name.
 *  prefix_group   device int32 [num_seqs]: the first sequence (leader) of each
 *                 sequence's group; a group's members are consecutive and its
 *                 leader names itself.  For member s with leader L, the
 *                 partitions that lie in the first min(shared_prefix_blocks[s],
 *                 shared_prefix_blocks[L]) entries and in full blocks of both
 *                 are read through L's table, so s's table must name the same
 *                 blocks there (else s's output is NaN).  An entry that does
 *                 not describe such a group (leader after s or negative, or
 *                 not its own leader) leaves s ungrouped: it is computed as by
 *                 pa_decode.
 *  max_group_size largest group (>= 1); it sets the members per workgroup.
 *  partition_size must be > 0 (the shared partitions are split-K partials).
 * A workgroup holds up to 4 query slots (members x query heads per kv head)
 * on the vector-ALU path and 16 on the matrix-core path (bf16 query,
 * head_dim 128, 4 or more query heads per kv head), so windows of up to
 * 4 / G or 16 / G members share a read (G = num_heads / num_kv_heads); where
 * fewer than two fit, the call computes exactly what pa_decode computes.  The
 * result equals pa_decode's bit for bit (same partitions, same order of
 * accumulation).
 */
int pa_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                            const int32_t* prefix_group, int max_group_size, int num_seqs,
                            int num_heads, int num_kv_heads, int head_dim, int block_size,
                            int max_blocks_per_seq, int64_t num_blocks, int max_context_len,
                            float scale, int partition_size, void* workspace,
                            size_t workspace_bytes, pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode_splitk_reduce -- merge the partition results pa_decode left in the
 * workspace: with M = max_p lse_p and w_p = exp(lse_p - M),
 * out = sum_p w_p o_p / sum_p w_p.  This is exact in real arithmetic: w_p is
 * partition p's share of the softmax denominator (up to the common factor
 * exp(M)), so the weighted mean of the partition means is the mean over all
 * keys.  The split-K merge of the long-context workload (see
 * pa_decode_workspace_bytes); the pages themselves have no split-K.  Sequences with at most one partition are
 * left untouched (pa_decode wrote them); when max_context_len <= partition_size
 * nothing is launched.  Arguments must match the pa_decode call that filled the
 * workspace (16-byte aligned).
 */
int pa_decode_splitk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                            const int32_t* context_lens, int num_seqs, int num_heads,
                            int head_dim, int max_context_len, int partition_size,
                            pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_decode_no_alloc -- pa_decode followed by pa_decode_splitk_reduce in one
 * call that allocates nothing and takes no workspace.  For callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * The split-K partials live in a fixed buffer of
 * pa_decode_no_alloc_scratch_bytes() (64 MiB) that the library holds on every
 * GPU it runs on until the process ends.  Arguments are pa_decode's without
 * the workspace; out receives the merged result.  A call whose partials
 * (pa_decode_workspace_bytes() of the same sizes) exceed the buffer returns
 * PA_ERR_SCRATCH and launches nothing; otherwise every pa_decode status
 * applies.  The first call on a device looks the buffer up on the current
 * device, so `stream` must belong to the current device.  All calls on one GPU
 * share the buffer: calls that overlap on one GPU (other streams, other host
 * threads) race on it, calls on one stream are ordered.  Nothing in the buffer
 * needs to start at zero.
 */
size_t pa_decode_no_alloc_scratch_bytes(void);
int pa_decode_no_alloc(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                       int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int64_t num_blocks,
                       int max_context_len, float scale, int partition_size, pa_dtype dtype,
                       hipStream_t stream);

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

/*
 * pa_prefill_chunk_split -- pa_prefill_chunk with the causal key range of long
 * query tiles split over several workgroups (split-K).
 *
 * A workgroup takes 128 query rows of one head; their keys (the paged prefix
 * and the chunk up to the tile's last row) are cut into runs of split_tokens
 * keys, each run one workgroup that leaves, per row, its normalised output
 * and the natural-log sum of exp(scale * q.k) over its keys in the workspace;
 * a merge launched by this call combines them by the log-sum-exp rule of
 * pa_decode_splitk_reduce.  Tiles whose range needs one run are written
 * directly.  The result equals pa_prefill_chunk's up to rounding; the point
 * is balance: a chunk over a long prefix no longer keeps one workgroup busy
 * long after the others (xdnf.cn article, section 六.4: chunks of one prompt
 * see everything before them).
 *
 *  max_context_len  upper bound on context_lens (sizes the workspace); a
 *                   longer sequence gets NaN rows.
 *  split_tokens     keys per run, a positive multiple of 64 (else PA_ERR_SHAPE).
 *  workspace        device buffer of at least pa_prefill_workspace_bytes(),
 *                   16-byte aligned (else PA_ERR_WORKSPACE): fp32 outputs
 *                   [num_query_tokens, num_heads, P, head_dim], then fp32 sums
 *                   [num_query_tokens, num_heads, P], P = ceil(max_context_len /
 *                   split_tokens).  The call overwrites what it needs of it.
 *  dtype            PA_BF16 only (the matrix-core kernel; PA_ERR_UNSUPPORTED
 *                   otherwise).
 * Every other argument as pa_prefill_chunk.
 */
size_t pa_prefill_workspace_bytes(int num_query_tokens, int num_heads, int head_dim,
                                  int max_context_len, int split_tokens);
int pa_prefill_chunk_split(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const int32_t* query_start_loc, const int32_t* context_lens,
                           int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks_per_seq,
                           int64_t num_blocks, int max_query_len, int max_context_len,
                           int split_tokens, float scale, void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, hipStream_t stream);

/*
 * FP8 KV cache.  The cache may store K and V as 8-bit floats (OCP E4M3: 1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, largest
 * magnitude 448), one byte per element, which halves the bytes decode streams
 * -- the resource decode is bound by (xdnf.cn article, section 六.5).  This
 * recasts the pages' suggestion of choosing a lower precision, fp8 among them,
 * for attention (intelliparadigm.com article, section 7.1) as a storage
 * format.  Each pool has one scale: a code c stands for value(c) * scale.
 * Pools are [num_blocks, num_kv_heads, block_size, head_dim] bytes, 4-byte
 * aligned; otherwise every convention above holds.
 */

/*
 * pa_reshape_and_cache_fp8 -- quantise each new token's K and V into its slot.
 *
 * As pa_reshape_and_cache, but key / value hold src_dtype values (fp32 or
 * bf16) and the caches receive, per element x, the code nearest to
 * fp32(x * fp32(1 / scale)) -- ties to the even code, magnitudes above 448
 * saturated to 448, NaN stored as 0x7F -- with k_scale for K and v_scale for
 * V.  The scales must be positive and finite (else PA_ERR_SHAPE).
 */
int pa_reshape_and_cache_fp8(const void* key, const void* value, uint8_t* key_cache,
                             uint8_t* value_cache, const int64_t* slot_mapping,
                             int64_t num_tokens, int64_t key_stride, int64_t value_stride,
                             int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                             pa_dtype src_dtype, float k_scale, float v_scale,
                             hipStream_t stream);

/*
 * pa_decode_fp8 -- pa_decode over FP8 caches: softmax(scale * q K^T) V with K
 * and V the values the codes stand for (code value times k_scale / v_scale).
 * query and out are dtype (fp32 or bf16); accumulation is fp32.  Split-K
 * partials use the same workspace layout, merged by pa_decode_splitk_reduce.
 * Supported groups: any group up to 16 for a bf16 query with head_dim 128
 * (grouped-query heads run on the matrix cores), else at most 4 query heads
 * per kv head (PA_ERR_UNSUPPORTED otherwise).  The scales must be positive
 * and finite (else PA_ERR_SHAPE).
 */
int pa_decode_fp8(void* out, const void* query, const uint8_t* key_cache,
                  const uint8_t* value_cache, const int32_t* block_tables,
                  const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                  int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int64_t num_blocks, int max_context_len, float scale,
                  float k_scale, float v_scale, int partition_size, void* workspace,
                  size_t workspace_bytes, pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode_fp8_shared_prefix -- pa_decode_shared_prefix over FP8 caches:
 * the arguments of pa_decode_fp8 plus prefix_group and max_group_size, with
 * the same grouping rules; equal bit for bit to pa_decode_fp8.
 */
int pa_decode_fp8_shared_prefix(void* out, const void* query, const uint8_t* key_cache,
                                const uint8_t* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                                const int32_t* prefix_group, int max_group_size, int num_seqs,
                                int num_heads, int num_kv_heads, int head_dim, int block_size,
                                int max_blocks_per_seq, int64_t num_blocks, int max_context_len,
                                float scale, float k_scale, float v_scale, int partition_size,
                                void* workspace, size_t workspace_bytes, pa_dtype dtype,
                                hipStream_t stream);

/*
 * pa_prefill_chunk_fp8 -- pa_prefill_chunk over FP8 caches: causal attention
 * of each sequence's chunk of new queries over its paged prefix and itself
 * (xdnf.cn article, section 六.4), with K and V the values the codes stand for
 * (code value times k_scale / v_scale), so that a step that mixes prefill
 * chunks with decode runs on one FP8 cache.  query and out are bf16 (the
 * matrix-core path; PA_ERR_UNSUPPORTED otherwise); accumulation is fp32.  The
 * scales must be positive and finite (else PA_ERR_SHAPE).  Every other
 * argument, and the NaN reporting of contract violations, as pa_prefill_chunk.
 */
int pa_prefill_chunk_fp8(void* out, const void* query, const uint8_t* key_cache,
                         const uint8_t* value_cache, const int32_t* block_tables,
                         const int32_t* query_start_loc, const int32_t* context_lens, int num_seqs,
                         int num_query_tokens, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int64_t num_blocks,
                         int max_query_len, float scale, float k_scale, float v_scale,
                         pa_dtype dtype, hipStream_t stream);

/*
 * pa_prefill_chunk_fp8_split -- pa_prefill_chunk_split over FP8 caches (the
 * arguments of pa_prefill_chunk_fp8 plus max_context_len, split_tokens and
 * the workspace, with the same rules).
 */
int pa_prefill_chunk_fp8_split(void* out, const void* query, const uint8_t* key_cache,
                               const uint8_t* value_cache, const int32_t* block_tables,
                               const int32_t* query_start_loc, const int32_t* context_lens,
                               int num_seqs, int num_query_tokens, int num_heads,
                               int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int64_t num_blocks, int max_query_len,
                               int max_context_len, int split_tokens, float scale, float k_scale,
                               float v_scale, void* workspace, size_t workspace_bytes,
                               pa_dtype dtype, hipStream_t stream);

/*
 * pa_copy_blocks -- copy whole physical blocks inside the K and V pools.
 *
 * For each pair (src, dst) = (block_mapping[2i], block_mapping[2i+1]) copies
 * block src of key_cache onto block dst, and the same in value_cache, bit for
 * bit.  This is the copy of copy-on-write: a sequence about to write into a
 * partly filled block it still shares gets its own copy first
 * (intelliparadigm.com article, sections 2.2 and 3.3).  The pairs
 * pa_bm_take_moves() hands out as copies are made for this call.
 *
 *  key_cache,
 *  value_cache    [num_blocks, num_kv_heads, block_size, head_dim], dtype (fp32, bf16 or
 *                 PA_FP8_E4M3 codes); updated in place.
 *  block_mapping  device int32 [num_pairs][2].
 * The pairs must be independent: destinations distinct and none of them a
 * source of the call (they run all at once).  A pair naming a block outside
 * [0, num_blocks), or with src == dst, is skipped.
 */
int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_mapping,
                   int64_t num_pairs, int num_kv_heads, int head_dim, int block_size,
                   int64_t num_blocks, pa_dtype dtype, hipStream_t stream);

/*
 * pa_swap_blocks -- copy whole blocks between two pools, one of them usually
 * in host memory: the swap space a sequence's blocks move to when it is
 * preempted and from which they return (intelliparadigm.com article, section
 * 5.1, swap space).
 *
 * For each pair (src, dst) copies block src of src_key / src_value onto block
 * dst of dst_key / dst_value, bit for bit.  When all four pools can be reached
 * by a kernel on the current device -- its own memory, or pinned host memory
 * (hipHostMalloc) that HIP maps at the same address -- one launch per 256 pairs
 * moves them (the pairs travel in the kernel arguments).  Otherwise (pageable
 * host memory, another device) the runtime copies them (hipMemcpyAsync, the
 * direction from the pointers), one copy per run of pairs whose sources and
 * destinations both advance by one, per pool.
 *
 *  src_key, src_value  [src_num_blocks, num_kv_heads, block_size, head_dim]
 *  dst_key, dst_value  [dst_num_blocks, num_kv_heads, block_size, head_dim]
 *  block_mapping       HOST int32 [num_pairs][2]; every id must be in range
 *                      (else PA_ERR_SHAPE and nothing is copied).
 * The pools must really hold the stated number of blocks.  Copies from or to
 * pageable memory are not asynchronous.  The pairs must be independent, as
 * for pa_copy_blocks.  A failed launch or copy returns PA_ERR_LAUNCH; moves
 * enqueued before it stay enqueued.
 */
int pa_swap_blocks(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                   const int32_t* block_mapping, int64_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int num_kv_heads, int head_dim, int block_size,
                   pa_dtype dtype, hipStream_t stream);

/*
 * Block manager -- host bookkeeping of which physical blocks hold which
 * sequence's tokens; it produces the block tables, context lengths and slot
 * mappings the kernels above take, and the block moves that keep them right.
 *
 * Model ("vLLM 基本原理", section PagedAttention, items 1-3, 按需分配 and 内存共享;
 * intelliparadigm.com article, sections 2.2, 2.3, 3.3 and 5.1; xdnf.cn article,
 * section 六.1):
 *  - a device pool of num_blocks blocks and a host pool (swap space) of
 *    num_host_blocks, each with a free stack and per-block reference counts;
 *  - a sequence (caller-chosen int64 id) owns a block table; it takes a new
 *    block only when its last block is full, so only the last block may be
 *    partly filled;
 *  - sharing: pa_bm_fork gives a new sequence every block of another (whole
 *    sequence), pa_bm_share chosen full blocks of another (a prefix, or any
 *    list of logical blocks); shared blocks count their holders;
 *  - copy on write: a sequence appending into a partly filled last block that
 *    others still hold gets a fresh block and a pending copy (old, new); the
 *    last holder writes in place;
 *  - a freed sequence returns its blocks at once; swap out / swap in move a
 *    sequence's blocks between the pools, each distinct block once per call.
 *
 * Policy: free blocks are a stack (the most recently released is reused
 * first; at the start ids come out in increasing order); a freed table is
 * released last entry first; every call is all-or-nothing -- on any error
 * nothing changes.
 *
 * Moves: copies (device -> device), swap-outs (device -> host) and swap-ins
 * (host -> device) accumulate as (src, dst) pairs until pa_bm_take_moves().
 * Until then a block named by a pending pair is not reused even if released,
 * and a call that would read a pending destination fails with PA_ERR_BUSY, so
 * the pairs of one take never overlap and may run in any order.
 *
 * The caller's step: free finished sequences, swap out / swap in, fork and
 * share, append slots (pa_bm_append_slots / pa_bm_append_batch), take the
 * moves and run them (pa_copy_blocks, pa_swap_blocks), then write the new
 * tokens' K/V into the slots (pa_reshape_and_cache) and run attention with
 * pa_bm_build_batch's tables.  A sequence that reserved slots since the last
 * take cannot be forked, shared from or swapped out (PA_ERR_BUSY): its new
 * tokens are not in its blocks yet.
 *
 * Not thread-safe: one caller thread per manager.  Block ids are int32, token
 * counts int64, slots int64 (block * block_size + row).
 */
typedef struct pa_block_manager pa_block_manager;

/* Creates a manager; *out is NULL on error.  block_size must be 16. */
int pa_bm_create(int64_t num_blocks, int64_t num_host_blocks, int block_size,
                 pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);
/* A new, empty resident sequence (PA_ERR_SEQ if the id exists). */
int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq);
/* Whole-sequence sharing: child starts with all of parent's tokens, on the same blocks. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
/* New sequence dst whose table is src's logical blocks logical_blocks[0..count-1], in that
 * order; each must be a full block of src (PA_ERR_SHAPE otherwise).  dst holds count *
 * block_size tokens.  0..n-1 shares a prefix of n blocks. */
int pa_bm_share(pa_block_manager* bm, int64_t src, int64_t dst, const int32_t* logical_blocks,
                int32_t count);
/* Releases the sequence's blocks (device or host) and forgets it. */
int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq);
/* Reserves count new token slots at the end of a resident sequence; slots (host, int64
 * [count]) receives them in token order.  May take new blocks and record copies. */
int pa_bm_append_slots(pa_block_manager* bm, int64_t seq, int32_t count, int64_t* slots);
/* pa_bm_append_slots for seqs[0..num_seqs-1] in order, slots back to back in slot_mapping
 * (host int64 [sum counts]).  Stops at the first sequence that fails and returns its status;
 * *num_done = sequences fully served (their slots are valid, the failed one changed nothing). */
int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs, const int32_t* counts,
                       int32_t num_seqs, int64_t* slot_mapping, int32_t* num_done);
/* Moves resident sequences to the host pool / swapped-out sequences back to the device. */
int pa_bm_swap_out(pa_block_manager* bm, const int64_t* seqs, int32_t count);
int pa_bm_swap_in(pa_block_manager* bm, const int64_t* seqs, int32_t count);
/* counts[0..2] = pending copies, swap-outs, swap-ins. */
int pa_bm_pending_moves(const pa_block_manager* bm, int64_t* counts);
/* Writes the pending pairs as int32 (src, dst) into host arrays of 2 * count entries each
 * (NULL allowed for an empty list), clears them and releases the blocks held back for them. */
int pa_bm_take_moves(pa_block_manager* bm, int32_t* copies, int32_t* swap_out, int32_t* swap_in);
int pa_bm_num_tokens(const pa_block_manager* bm, int64_t seq, int64_t* num_tokens);
int pa_bm_is_swapped(const pa_block_manager* bm, int64_t seq, int32_t* swapped);
/* Copies the table (device ids if resident, host ids if swapped out) into table[capacity];
 * *length is set even when capacity is too small (then PA_ERR_SHAPE). */
int pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* table, int32_t capacity,
                      int32_t* length);
/* Free blocks of the device pool (host == 0) or the host pool; negative status on error. */
int64_t pa_bm_num_free(const pa_block_manager* bm, int host);
/* Attention inputs for resident sequences seqs[0..num_seqs-1], into host arrays:
 * block_tables int32 [num_seqs, max_blocks_per_seq] (unused entries -1), context_lens int32
 * [num_seqs], and optionally shared_prefix_blocks int32 [num_seqs] = leading table entries
 * whose block another sequence also holds (pa_decode's cache hint). */
int pa_bm_build_batch(const pa_block_manager* bm, const int64_t* seqs, int32_t num_seqs,
                      int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens,
                      int32_t* shared_prefix_blocks);
/* Sharing groups of a decode batch for pa_decode_shared_prefix, over resident sequences
 * seqs[0..num_seqs-1] in batch order (host arrays of num_seqs entries).  A group is a run of
 * consecutive entries whose tables start with the same physical block as the run's first entry
 * -- samples forked from one prompt ("vLLM 基本原理", section 内存共享), or requests on one cached
 * prefix (xdnf.cn article, section 六.3) -- so the caller places sharers next to each other.
 * prefix_group[i] = index of the run's first entry; group_blocks[i] = for a member, its leading
 * table entries equal to the first entry's, for the first entry the largest of its members'
 * counts (0 in a group of one).  Pass group_blocks as pa_decode_shared_prefix's
 * shared_prefix_blocks; *max_group_size (optional) receives the largest run. */
int pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seqs, int32_t num_seqs,
                        int32_t* prefix_group, int32_t* group_blocks, int32_t* max_group_size);
/* Checks the invariants (reference counts = table occurrences, free + held-back blocks =
 * unreferenced ones, table lengths = ceil(tokens / block_size), cache entries consistent):
 * PA_OK or PA_ERR_STATE. */
int pa_bm_check(const pa_block_manager* bm);

/*
 * Prefix cache.  Requests that share a prefix -- a system prompt, a fixed
 * document, few-shot examples, earlier turns -- reuse its KV blocks and skip
 * their prefill (xdnf.cn article, section 六.3).  A hit needs the same model,
 * precision, quantisation and adapter (the caller folds them into `salt`), the
 * same tokens from position 0, and whole blocks: a partly filled tail is never
 * reused.
 *
 *  - Key of full block j: FNV-1a 64 over (key of block j-1, or 0 for j = 0;
 *    salt; the block's 16 token ids), each as little-endian bytes (8, 8, 4 x 16).
 *  - A sequence created from a prompt, or forked from one, knows its tokens;
 *    each of its blocks that fills (pa_bm_append_tokens) enters the cache when
 *    the batch ends (pa_bm_take_moves), if the sequence still holds it -- its
 *    tokens are then about to be written.
 *  - A hit is verified exactly, not by the key: same salt, same 16 tokens, and
 *    a parent that is the block matched just before (none for block 0).  A key
 *    whose entry fails that check is taken over by the newly filled block.
 *  - Cached blocks nobody holds stay cached.  Allocation takes idle blocks
 *    without cached contents first, then evicts the cached block that has
 *    been idle longest.  Blocks brought back by a swap-in, and sequences made
 *    by pa_bm_share or pa_bm_add_sequence, are never entered.
 */
/* keys[j] = key of full block j of tokens[0..num_tokens-1] (num_tokens / 16 keys). */
int pa_bm_prefix_keys(const int32_t* tokens, int64_t num_tokens, uint64_t salt, uint64_t* keys);
/* New sequence for a prompt: it starts on the longest cached prefix of whole blocks, at most
 * the blocks before the prompt's last token (which is always left to compute), and
 * *num_cached_tokens says how many tokens that covers.  Append the rest of the prompt with
 * pa_bm_append_tokens; prefill only those. */
int pa_bm_add_prompt(pa_block_manager* bm, int64_t seq, const int32_t* tokens,
                     int64_t num_tokens, uint64_t salt, int64_t* num_cached_tokens);
/* pa_bm_append_slots for a sequence that knows its tokens, with their ids (PA_ERR_SEQ for a
 * sequence that does not). */
int pa_bm_append_tokens(pa_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t count,
                        int64_t* slots);
/* Cache entries (blocks that can be hit); negative status on error. */
int64_t pa_bm_num_cached_blocks(const pa_block_manager* bm);

/*
 * pa_sample -- draw the next token of each row: temperature, top-k, top-p,
 * then a draw from what is left, fused in one kernel with no sort ("vLLM
 * 基本原理", section FlashInfer 采样器: temperature scaling, top-k keeps the K
 * most probable tokens, top-p the most probable ones whose cumulative
 * probability reaches P, the next token is drawn from the rest).
 *
 * For row r: z = logits[r] / temperature[r] (NaN counts as -inf).  If
 * 0 < top_k[r] < vocab_size, tokens whose z is below the top_k[r]-th largest
 * are dropped (ties with it stay).  Then, on the probabilities renormalised over
 * the rest, a token stays if the mass of the tokens strictly more probable than
 * it is below top_p[r] (top_p[r] = 1 keeps all).  tokens[r] is the first token,
 * in vocabulary order, at which the cumulative probability of what stayed
 * exceeds uniform[r]: the inverse of the distribution function, so the draw is
 * a deterministic function of the caller's uniform number.  Weights
 * exp(z - max z) are kept in fixed point with 32 fraction bits (64-bit integer
 * sums, exact in any order): a token more than 2^32 times less likely than
 * the most likely one counts as probability zero and takes no part in top-k.
 *
 *  tokens       device int32 [num_rows]: the drawn token, or -1 for a row with
 *               no finite logit or out-of-range parameters (temperature <= 0,
 *               top_p outside (0, 1], uniform outside [0, 1)).
 *  logits       device [num_rows, row_stride], dtype fp32 or bf16; vocab_size
 *               <= 32768 (the row is held in registers), else PA_ERR_UNSUPPORTED.
 *  temperature, top_p, uniform  device float [num_rows]; top_k device int32 [num_rows].
 */
int pa_sample(int32_t* tokens, const void* logits, int64_t row_stride, int num_rows,
              int vocab_size, const float* temperature, const int32_t* top_k,
              const float* top_p, const float* uniform, pa_dtype dtype, hipStream_t stream);

/*
 * Measurement aid (not an operation of the method): the HBM read rate this
 * part reaches with plain, fully coalesced 16-byte loads, the ceiling the
 * decode kernels -- bound by HBM reads (xdnf.cn article, section 六.5) -- are
 * compared with.
 *
 * pa_stream_read reads every byte of `buffer` once (nontemporal 16-byte
 * loads, grid-stride) and writes pa_stream_read_sink_words() 32-bit words to
 * `sink`, one per workgroup; their XOR equals the XOR of the buffer's 32-bit
 * words.
 *  buffer  device memory, 16-byte aligned; bytes a multiple of 16 (else
 *          PA_ERR_SHAPE).  0 bytes writes zeros to the sink.
 *  sink    device uint32 [pa_stream_read_sink_words()].
 */
int pa_stream_read_sink_words(void);
int pa_stream_read(const void* buffer, int64_t bytes, uint32_t* sink, hipStream_t stream);

/* Human-readable name of a pa_status value (static storage). */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
