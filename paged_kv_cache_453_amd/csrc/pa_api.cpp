// C ABI of the paged-attention library: argument checks, kernel choice, launch.
//
// Every scalar and pointer argument is checked here, on the host, before any
// HIP call; a bad argument returns a negative pa_status and launches nothing.
// Launches go to the caller's stream; nothing here allocates or synchronises.
#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"
#include "pa_launch.h"

namespace {

constexpr int kBlockSize = 16;
constexpr int kPrefillKeyTile = 64;   // keys per prefill tile: split runs are whole tiles
constexpr int kMaxGroup = 16;
constexpr int64_t kMaxGridY = 65535;

bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(pa_dtype t) { return t == PA_F32 || t == PA_BF16; }
bool pool_dtype_ok(pa_dtype t) { return dtype_ok(t) || t == PA_FP8_E4M3; }
int elem_bytes(pa_dtype t) { return t == PA_F32 ? 4 : t == PA_BF16 ? 2 : 1; }

int max_partitions(int max_context_len, int partition_size) {
  if (partition_size <= 0) return 1;
  const int p = (int)(((int64_t)max_context_len + partition_size - 1) / partition_size);
  return p > 0 ? p : 1;
}

int status_of(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

bool scale_ok(float s) { return s > 0.f && s < INFINITY; }
// The split-K merge reads the partials in 16-byte pieces.
bool workspace_ok(const void* ws, size_t bytes, size_t need) {
  return ws && bytes >= need && (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
}

// The scalar and pointer checks of every decode entry point, workspace aside.
int decode_check(const void* out, const void* query, const void* key_cache,
                 const void* value_cache, const int32_t* block_tables,
                 const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                 const int32_t* prefix_group, int max_group_size, int num_seqs, int num_heads,
                 int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                 int64_t num_blocks, int max_context_len, int partition_size, pa_dtype dtype,
                 bool fp8, float k_scale, float v_scale) {
  if (num_seqs < 0) return PA_ERR_SHAPE;
  if (prefix_group != nullptr) {
    // the grouped pass writes split-K partials and needs the shared counts
    if (num_seqs > 0 && !shared_prefix_blocks) return PA_ERR_NULL;
    if (partition_size <= 0 || max_group_size < 1) return PA_ERR_SHAPE;
  }
  if (num_seqs > 0 && (!out || !query || !key_cache || !value_cache || !block_tables ||
                       !context_lens))
    return PA_ERR_NULL;
  if (!dtype_ok(dtype) || block_size != kBlockSize || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 ||
      num_kv_heads > kMaxGridY || max_blocks_per_seq < 1 || num_blocks < 1 ||
      max_context_len < 0 || partition_size < 0 || partition_size % kBlockSize != 0)
    return PA_ERR_SHAPE;
  if (fp8 && (!scale_ok(k_scale) || !scale_ok(v_scale))) return PA_ERR_SHAPE;
  const int group = num_heads / num_kv_heads;
  if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (fp8 && !pa::decode_fp8_supported(group, head_dim, dtype == PA_BF16))
    return PA_ERR_UNSUPPORTED;
  const int nparts = max_partitions(max_context_len, partition_size);
  if (nparts > kMaxGridY || (int64_t)num_seqs * num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

// Shared by pa_decode and pa_decode_fp8: checks, then the kernel choice.
int decode_impl(void* out, const void* query, const void* key_cache, const void* value_cache,
                const int32_t* block_tables, const int32_t* context_lens,
                const int32_t* shared_prefix_blocks, const int32_t* prefix_group,
                int max_group_size, int num_seqs, int num_heads,
                int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                int64_t num_blocks, int max_context_len, float scale, int partition_size,
                void* workspace, size_t workspace_bytes, pa_dtype dtype, bool fp8,
                float k_scale, float v_scale, hipStream_t stream) {
  const int st = decode_check(out, query, key_cache, value_cache, block_tables, context_lens,
                              shared_prefix_blocks, prefix_group, max_group_size, num_seqs,
                              num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              num_blocks, max_context_len, partition_size, dtype, fp8, k_scale,
                              v_scale);
  if (st != PA_OK) return st;
  const int group = num_heads / num_kv_heads;
  const int nparts = max_partitions(max_context_len, partition_size);
  if (partition_size > 0) {
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                  partition_size);
    if (num_seqs > 0 && !workspace_ok(workspace, workspace_bytes, need)) return PA_ERR_WORKSPACE;
  }
  if (num_seqs == 0) return PA_OK;
  pa::DecodeArgs a = {};
  a.out = out;
  a.query = query;
  a.k_cache = key_cache;
  a.v_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = nullptr;
  a.shared_prefix_blocks = shared_prefix_blocks;
  // The launchers size the windows of sharers per grouped workgroup from
  // max_group_size and the query slots their kernel holds; with fewer than two
  // members per window the call is a plain decode.
  a.prefix_group = prefix_group;
  a.group_members = prefix_group ? max_group_size : 0;
  const size_t rows = (size_t)num_seqs * num_heads * nparts;
  a.part_o = partition_size > 0 ? static_cast<float*>(workspace) : nullptr;
  a.part_lse = partition_size > 0 ? static_cast<float*>(workspace) + rows * head_dim : nullptr;
  a.sched = partition_size > 0 ? reinterpret_cast<int*>(a.part_lse + rows) : nullptr;
  a.num_seqs = num_seqs;
  a.num_items = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_blocks = partition_size / kBlockSize;
  a.max_partitions = nparts;
  a.max_query_len = 1;
  a.scale_log2 = (fp8 ? scale * k_scale : scale) * 1.4426950408889634f;
  a.v_scale = fp8 ? v_scale : 1.f;
  if (fp8) return status_of(pa::launch_decode_fp8(a, head_dim, dtype == PA_BF16, stream));
  return status_of(pa::launch_decode(a, head_dim, dtype == PA_BF16, stream));
}

}  // namespace

namespace pa {
int check_decode_args(const void* out, const void* query, const void* key_cache,
                      const void* value_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, int max_blocks_per_seq, int64_t num_blocks,
                      int max_context_len, int partition_size, pa_dtype dtype) {
  return decode_check(out, query, key_cache, value_cache, block_tables, context_lens, nullptr,
                      nullptr, 0, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, num_blocks, max_context_len, partition_size, dtype,
                      false, 1.f, 1.f);
}
}  // namespace pa

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer argument";
    case PA_ERR_SHAPE: return "invalid or inconsistent size argument";
    case PA_ERR_UNSUPPORTED: return "unsupported block_size, head_dim, dtype or group size";
    case PA_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case PA_ERR_LAUNCH: return "kernel launch or copy failed";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    case PA_ERR_SEQ: return "unknown or duplicate sequence, or wrong side of a swap";
    case PA_ERR_BUSY: return "pending block moves must be taken and run first";
    case PA_ERR_NO_MEMORY: return "host allocation failed";
    case PA_ERR_STATE: return "block manager invariant violated";
    case PA_ERR_SCRATCH:
      return "split-K partials larger than the fixed buffer of pa_decode_no_alloc "
             "(pa_decode_no_alloc_scratch_bytes())";
    default: return "unknown status";
  }
}

int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int64_t key_stride,
                         int64_t value_stride, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, pa_dtype dtype, hipStream_t stream) {
  if (!key_cache || !value_cache) return PA_ERR_NULL;
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_NULL;
  if (!dtype_ok(dtype) || block_size != kBlockSize || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_tokens > INT32_MAX || num_kv_heads < 1 || num_blocks < 1)
    return PA_ERR_SHAPE;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (key_stride < row || value_stride < row) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  pa::ScatterArgs a = {};
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.elem_bytes = elem_bytes(dtype);
  a.fp8 = false;
  return status_of(pa::launch_reshape_and_cache(a, stream));
}

int pa_reshape_and_cache_fp8(const void* key, const void* value, uint8_t* key_cache,
                             uint8_t* value_cache, const int64_t* slot_mapping,
                             int64_t num_tokens, int64_t key_stride, int64_t value_stride,
                             int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                             pa_dtype src_dtype, float k_scale, float v_scale,
                             hipStream_t stream) {
  if (!key_cache || !value_cache) return PA_ERR_NULL;
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_NULL;
  if (!dtype_ok(src_dtype) || block_size != kBlockSize || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) & 3) != 0)
    return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_tokens > INT32_MAX || num_kv_heads < 1 || num_blocks < 1)
    return PA_ERR_SHAPE;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (key_stride < row || value_stride < row) return PA_ERR_SHAPE;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  pa::ScatterArgs a = {};
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.elem_bytes = elem_bytes(src_dtype);
  a.fp8 = true;
  a.k_inv_scale = 1.f / k_scale;
  a.v_inv_scale = 1.f / v_scale;
  return status_of(pa::launch_reshape_and_cache(a, stream));
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                 int partition_size) {
  if (partition_size <= 0 || num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return 0;
  const size_t nparts = (size_t)max_partitions(max_context_len, partition_size);
  const size_t rows = (size_t)num_seqs * (size_t)num_heads * nparts;
  const size_t sched = (size_t)pa::sched_ints(num_seqs, (int64_t)nparts);
  return rows * (size_t)head_dim * sizeof(float) + rows * sizeof(float) + sched * sizeof(int);
}

int pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* context_lens,
              const int32_t* shared_prefix_blocks, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int64_t num_blocks, int max_context_len, float scale,
              int partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
              hipStream_t stream) {
  return decode_impl(out, query, key_cache, value_cache, block_tables, context_lens,
                     shared_prefix_blocks, nullptr, 0, num_seqs, num_heads, num_kv_heads,
                     head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, dtype, false, 1.f, 1.f, stream);
}

int pa_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                            const int32_t* prefix_group, int max_group_size, int num_seqs,
                            int num_heads, int num_kv_heads, int head_dim, int block_size,
                            int max_blocks_per_seq, int64_t num_blocks, int max_context_len,
                            float scale, int partition_size, void* workspace,
                            size_t workspace_bytes, pa_dtype dtype, hipStream_t stream) {
  if (num_seqs > 0 && !prefix_group) return PA_ERR_NULL;
  return decode_impl(out, query, key_cache, value_cache, block_tables, context_lens,
                     shared_prefix_blocks, prefix_group, max_group_size, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                     false, 1.f, 1.f, stream);
}

int pa_decode_fp8(void* out, const void* query, const uint8_t* key_cache,
                  const uint8_t* value_cache, const int32_t* block_tables,
                  const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                  int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int64_t num_blocks, int max_context_len, float scale,
                  float k_scale, float v_scale, int partition_size, void* workspace,
                  size_t workspace_bytes, pa_dtype dtype, hipStream_t stream) {
  return decode_impl(out, query, key_cache, value_cache, block_tables, context_lens,
                     shared_prefix_blocks, nullptr, 0, num_seqs, num_heads, num_kv_heads,
                     head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, dtype, true, k_scale, v_scale,
                     stream);
}

int pa_decode_fp8_shared_prefix(void* out, const void* query, const uint8_t* key_cache,
                                const uint8_t* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                                const int32_t* prefix_group, int max_group_size, int num_seqs,
                                int num_heads, int num_kv_heads, int head_dim, int block_size,
                                int max_blocks_per_seq, int64_t num_blocks, int max_context_len,
                                float scale, float k_scale, float v_scale, int partition_size,
                                void* workspace, size_t workspace_bytes, pa_dtype dtype,
                                hipStream_t stream) {
  if (num_seqs > 0 && !prefix_group) return PA_ERR_NULL;
  return decode_impl(out, query, key_cache, value_cache, block_tables, context_lens,
                     shared_prefix_blocks, prefix_group, max_group_size, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                     true, k_scale, v_scale, stream);
}

int pa_decode_splitk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                            const int32_t* context_lens, int num_seqs, int num_heads,
                            int head_dim, int max_context_len, int partition_size,
                            pa_dtype out_dtype, hipStream_t stream) {
  if (num_seqs < 0) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!out || !context_lens)) return PA_ERR_NULL;
  if (!dtype_ok(out_dtype) || !head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_heads < 1 || num_heads > kMaxGridY || max_context_len < 0 || partition_size <= 0 ||
      partition_size % kBlockSize != 0 || (int64_t)num_seqs * num_heads > INT32_MAX)
    return PA_ERR_SHAPE;
  const size_t need =
      pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size);
  if (num_seqs > 0 && !workspace_ok(workspace, workspace_bytes, need)) return PA_ERR_WORKSPACE;
  if (num_seqs == 0) return PA_OK;
  const int nparts = max_partitions(max_context_len, partition_size);
  if (nparts <= 1) return PA_OK;   // every sequence has one partition: pa_decode wrote it
  const size_t rows = (size_t)num_seqs * num_heads * nparts;
  pa::ReduceArgs a;
  a.out = out;
  a.part_o = static_cast<const float*>(workspace);
  a.part_lse = static_cast<const float*>(workspace) + rows * head_dim;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.max_partitions = nparts;
  a.partition_tokens = partition_size;
  a.max_context_len = max_context_len;
  return status_of(pa::launch_splitk_reduce(a, head_dim, out_dtype == PA_BF16, stream));
}

namespace {

int prefill_impl(void* out, const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* query_start_loc,
                 const int32_t* context_lens, int num_seqs, int num_query_tokens, int num_heads,
                 int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                 int64_t num_blocks, int max_query_len, float scale, bool fp8, float k_scale,
                 float v_scale, pa_dtype dtype, hipStream_t stream, int split_tokens = 0,
                 int max_context_len = 0, void* workspace = nullptr, size_t workspace_bytes = 0) {
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0) return PA_ERR_SHAPE;
  if (split_tokens < 0 || split_tokens % kPrefillKeyTile != 0 ||
      (split_tokens > 0 && max_context_len < 0))
    return PA_ERR_SHAPE;
  if (split_tokens > 0 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;   // matrix-core path
  if (num_seqs > 0 && (!out || !query || !key_cache || !value_cache || !block_tables ||
                       !query_start_loc || !context_lens))
    return PA_ERR_NULL;
  if (!dtype_ok(dtype) || block_size != kBlockSize || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (fp8 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;   // the matrix-core path only
  if (fp8 && (!scale_ok(k_scale) || !scale_ok(v_scale))) return PA_ERR_SHAPE;
  if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 ||
      num_heads > kMaxGridY || num_kv_heads > kMaxGridY || max_blocks_per_seq < 1 ||
      num_blocks < 1 || num_seqs > kMaxGridY)
    return PA_ERR_SHAPE;
  if (num_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_query_tokens * num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  const int nsplit = split_tokens > 0 ? max_partitions(max_context_len, split_tokens) : 1;
  if (split_tokens > 0) {
    if (nsplit > kMaxGridY) return PA_ERR_SHAPE;
    const size_t need = pa_prefill_workspace_bytes(num_query_tokens, num_heads, head_dim,
                                                   max_context_len, split_tokens);
    if (num_seqs > 0 && num_query_tokens > 0 && !workspace_ok(workspace, workspace_bytes, need))
      return PA_ERR_WORKSPACE;
  }
  if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
  pa::DecodeArgs a = {};
  a.out = out;
  a.query = query;
  a.k_cache = key_cache;
  a.v_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  if (split_tokens > 0) {
    const size_t rows = (size_t)num_query_tokens * num_heads * nsplit;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = static_cast<float*>(workspace) + rows * head_dim;
  }
  a.shared_prefix_blocks = nullptr;
  a.num_seqs = num_seqs;
  a.num_items = num_query_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = split_tokens > 0 ? max_context_len : INT_MAX;
  a.partition_blocks = split_tokens / kBlockSize;
  a.max_partitions = nsplit;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * (fp8 ? k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = fp8 ? v_scale : 1.f;
  if (fp8) return status_of(pa::launch_prefill_mfma_fp8(a, head_dim, stream));
  if (dtype == PA_BF16) return status_of(pa::launch_prefill_mfma(a, head_dim, stream));
  return status_of(pa::launch_decode(a, head_dim, false, stream));
}

}  // namespace

int pa_prefill_chunk(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* query_start_loc,
                     const int32_t* context_lens, int num_seqs, int num_query_tokens,
                     int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int64_t num_blocks, int max_query_len, float scale,
                     pa_dtype dtype, hipStream_t stream) {
  return prefill_impl(out, query, key_cache, value_cache, block_tables, query_start_loc,
                      context_lens, num_seqs, num_query_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_query_len, scale, false, 1.f,
                      1.f, dtype, stream);
}

int pa_prefill_chunk_fp8(void* out, const void* query, const uint8_t* key_cache,
                         const uint8_t* value_cache, const int32_t* block_tables,
                         const int32_t* query_start_loc, const int32_t* context_lens, int num_seqs,
                         int num_query_tokens, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int64_t num_blocks,
                         int max_query_len, float scale, float k_scale, float v_scale,
                         pa_dtype dtype, hipStream_t stream) {
  return prefill_impl(out, query, key_cache, value_cache, block_tables, query_start_loc,
                      context_lens, num_seqs, num_query_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_query_len, scale, true,
                      k_scale, v_scale, dtype, stream);
}

size_t pa_prefill_workspace_bytes(int num_query_tokens, int num_heads, int head_dim,
                                  int max_context_len, int split_tokens) {
  if (split_tokens <= 0 || num_query_tokens <= 0 || num_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return 0;
  const size_t rows = (size_t)num_query_tokens * (size_t)num_heads *
                      (size_t)max_partitions(max_context_len, split_tokens);
  return rows * (size_t)head_dim * sizeof(float) + rows * sizeof(float);
}

int pa_prefill_chunk_split(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const int32_t* query_start_loc, const int32_t* context_lens,
                           int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks_per_seq,
                           int64_t num_blocks, int max_query_len, int max_context_len,
                           int split_tokens, float scale, void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, hipStream_t stream) {
  if (split_tokens <= 0) return PA_ERR_SHAPE;
  return prefill_impl(out, query, key_cache, value_cache, block_tables, query_start_loc,
                      context_lens, num_seqs, num_query_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_query_len, scale, false, 1.f,
                      1.f, dtype, stream, split_tokens, max_context_len, workspace,
                      workspace_bytes);
}

int pa_prefill_chunk_fp8_split(void* out, const void* query, const uint8_t* key_cache,
                               const uint8_t* value_cache, const int32_t* block_tables,
                               const int32_t* query_start_loc, const int32_t* context_lens,
                               int num_seqs, int num_query_tokens, int num_heads,
                               int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int64_t num_blocks, int max_query_len,
                               int max_context_len, int split_tokens, float scale, float k_scale,
                               float v_scale, void* workspace, size_t workspace_bytes,
                               pa_dtype dtype, hipStream_t stream) {
  if (split_tokens <= 0) return PA_ERR_SHAPE;
  return prefill_impl(out, query, key_cache, value_cache, block_tables, query_start_loc,
                      context_lens, num_seqs, num_query_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_query_len, scale, true,
                      k_scale, v_scale, dtype, stream, split_tokens, max_context_len, workspace,
                      workspace_bytes);
}

int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_mapping,
                   int64_t num_pairs, int num_kv_heads, int head_dim, int block_size,
                   int64_t num_blocks, pa_dtype dtype, hipStream_t stream) {
  if (!key_cache || !value_cache) return PA_ERR_NULL;
  if (num_pairs > 0 && !block_mapping) return PA_ERR_NULL;
  if (!pool_dtype_ok(dtype) || block_size != kBlockSize || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_kv_heads < 1 || num_blocks < 1) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  pa::BlockPools p;
  p.src_k = p.dst_k = key_cache;
  p.src_v = p.dst_v = value_cache;
  p.block_bytes = (int64_t)num_kv_heads * kBlockSize * head_dim * elem_bytes(dtype);
  p.src_blocks = p.dst_blocks = num_blocks;
  p.num_pairs = num_pairs;
  return status_of(pa::launch_copy_blocks(p, block_mapping, stream));
}

}  // extern "C"

namespace {

// Whether a kernel on the current device may read and write [p, p + bytes):
// device memory of this device, or pinned host memory that HIP maps at the
// same address for the device.  Anything else (pageable host memory, another
// device, memory HIP does not know) is left to the runtime's copies.
bool kernel_reachable(const void* p, int64_t bytes) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const char* ends[2] = {static_cast<const char*>(p), static_cast<const char*>(p) + bytes - 1};
  for (const char* q : ends) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, q) != hipSuccess) {
      (void)hipGetLastError();   // an unknown pointer is an answer here, not an error
      return false;
    }
    if (at.type == hipMemoryTypeDevice) {
      if (at.device != dev) return false;
    } else if (at.type == hipMemoryTypeHost) {
      if (at.devicePointer != q) return false;
    } else {
      return false;
    }
  }
  return true;
}

}  // namespace

extern "C" {

int pa_swap_blocks(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                   const int32_t* block_mapping, int64_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int num_kv_heads, int head_dim, int block_size,
                   pa_dtype dtype, hipStream_t stream) {
  if (!src_key || !src_value || !dst_key || !dst_value) return PA_ERR_NULL;
  if (num_pairs > 0 && !block_mapping) return PA_ERR_NULL;
  if (!pool_dtype_ok(dtype) || block_size != kBlockSize || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_kv_heads < 1 || src_num_blocks < 1 || dst_num_blocks < 1)
    return PA_ERR_SHAPE;
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int32_t s = block_mapping[2 * i], d = block_mapping[2 * i + 1];
    if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) return PA_ERR_SHAPE;
  }
  if (num_pairs == 0) return PA_OK;
  const int64_t bb = (int64_t)num_kv_heads * kBlockSize * head_dim * elem_bytes(dtype);
  const int64_t src_bytes = src_num_blocks * bb, dst_bytes = dst_num_blocks * bb;
  if (kernel_reachable(src_key, src_bytes) && kernel_reachable(src_value, src_bytes) &&
      kernel_reachable(dst_key, dst_bytes) && kernel_reachable(dst_value, dst_bytes)) {
    pa::BlockPools p;
    p.src_k = src_key;
    p.src_v = src_value;
    p.dst_k = dst_key;
    p.dst_v = dst_value;
    p.block_bytes = bb;
    p.src_blocks = src_num_blocks;
    p.dst_blocks = dst_num_blocks;
    p.num_pairs = num_pairs;
    return status_of(pa::launch_swap_blocks(p, block_mapping, stream));
  }
  const char* sk = static_cast<const char*>(src_key);
  const char* sv = static_cast<const char*>(src_value);
  char* dk = static_cast<char*>(dst_key);
  char* dv = static_cast<char*>(dst_value);
  for (int64_t i = 0; i < num_pairs;) {
    // merge the run of pairs whose source and destination both advance by one
    const int64_t s0 = block_mapping[2 * i], d0 = block_mapping[2 * i + 1];
    int64_t n = 1;
    while (i + n < num_pairs && block_mapping[2 * (i + n)] == s0 + n &&
           block_mapping[2 * (i + n) + 1] == d0 + n)
      ++n;
    if (hipMemcpyAsync(dk + d0 * bb, sk + s0 * bb, n * bb, hipMemcpyDefault, stream) !=
            hipSuccess ||
        hipMemcpyAsync(dv + d0 * bb, sv + s0 * bb, n * bb, hipMemcpyDefault, stream) != hipSuccess)
      return PA_ERR_LAUNCH;
    i += n;
  }
  return PA_OK;
}

int pa_sample(int32_t* tokens, const void* logits, int64_t row_stride, int num_rows,
              int vocab_size, const float* temperature, const int32_t* top_k,
              const float* top_p, const float* uniform, pa_dtype dtype, hipStream_t stream) {
  if (num_rows < 0) return PA_ERR_SHAPE;
  if (num_rows > 0 && (!tokens || !logits || !temperature || !top_k || !top_p || !uniform))
    return PA_ERR_NULL;
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (vocab_size < 1 || row_stride < vocab_size) return PA_ERR_SHAPE;
  if (vocab_size > pa::kMaxSampleVocab) return PA_ERR_UNSUPPORTED;
  if (num_rows == 0) return PA_OK;
  pa::SampleArgs a;
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = vocab_size;
  a.num_rows = num_rows;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.uniform = uniform;
  a.tokens = tokens;
  return status_of(pa::launch_sample(a, dtype == PA_BF16, stream));
}

int pa_stream_read_sink_words(void) { return pa::kStreamBlocks; }

int pa_stream_read(const void* buffer, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0) return PA_ERR_SHAPE;
  if (!sink || (bytes > 0 && !buffer)) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buffer) & 15) != 0) return PA_ERR_SHAPE;
  return status_of(pa::launch_stream_read(buffer, bytes, sink, stream));
}

}  // extern "C"
