// Host-side launchers of the paged-attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

struct ScatterArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t key_stride;     // elements between tokens
  int64_t value_stride;
  int num_kv_heads;
  int head_dim;
  int64_t num_blocks;
  int elem_bytes;         // of key/value (and of the caches, unless FP8)
  // FP8 caches: codes = E4M3(x * inv_scale), x widened to fp32 from key/value
  bool fp8;
  float k_inv_scale;
  float v_inv_scale;
};

struct DecodeArgs {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;  // non-null: one work item per prefill query token
  const int32_t* shared_prefix_blocks;  // optional per-sequence cache hint (decode only)
  // Decode only, optional: prefix_group[s] = first sequence of s's sharing
  // group.  Windows of group_members (>= 2) consecutive members read their
  // common full partitions once, in the grouped pass (decode_groups.h); the
  // entry point passes the caller's largest group size, each launcher the
  // window size its kernel holds.
  const int32_t* prefix_group;
  int group_members;
  float* part_o;
  float* part_lse;
  // Split-K decode only: the schedule of the dealt decode (null: none).
  int* sched;
  int num_seqs;
  int num_items;          // grid z: sequences (decode) or query tokens (prefill)
  int num_heads;
  int num_kv_heads;
  int group;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int partition_blocks;   // 0 = one workgroup walks the whole context
  int max_partitions;
  int max_query_len;
  float scale_log2;       // softmax scale * log2(e) (times the K scale for FP8 caches)
  float v_scale;          // FP8 caches: the V scale, applied to the output
};

// The split-K schedule of the dealt decode (decode_schedule_kernel), in ints:
// the number of (sequence, partition) pairs with work; from kSchedHeader on,
// num_seqs * max_partitions slots holding those pairs (sequence *
// max_partitions + partition), longest partition first.
constexpr int kSchedPairs = 0;
constexpr int kSchedHeader = 64;

inline int64_t sched_ints(int64_t num_seqs, int64_t nparts) {
  return kSchedHeader + num_seqs * nparts;
}

// The deal of the dealt decode's units (in the schedule's order) to the XCDs:
// every period of kDealPeriod units gives kDealRounds to each XCD in turn,
// then kDealExtra more to each even-numbered one.  Workgroup ids reach the
// XCDs round-robin (XCD b % 8), and each XCD runs its workgroups in order of
// b / 8, so workgroup b takes XCD b % 8's (b / 8)-th unit.
constexpr int kXcds = 8;   // accelerator dies (XCDs): workgroup ids go to them round-robin
constexpr int kDealRounds = 6;
constexpr int kDealExtra = 1;
constexpr int kDealPeriod = kXcds * kDealRounds + (kXcds / 2) * kDealExtra;

__host__ __device__ inline int dealt_unit(int b) {
  const int x = b % kXcds;
  const int j = b / kXcds;
  const int n = (x & 1) ? kDealRounds : kDealRounds + kDealExtra;
  const int q = j / n;
  const int k = j - q * n;
  const int p = k < kDealRounds ? k * kXcds + x
                                : kXcds * kDealRounds + (k - kDealRounds) * (kXcds / 2) + x / 2;
  return q * kDealPeriod + p;
}

// Workgroups of a dealt launch that covers `units` units: every XCD's slots
// for the periods they span, at the larger share.
inline int64_t deal_blocks(int64_t units) {
  return kXcds * ((units + kDealPeriod - 1) / kDealPeriod) * (kDealRounds + kDealExtra);
}

// Query slots (sharing members x query heads per kv head) of one grouped-pass
// workgroup: its registers hold that many accumulators, and 4 keeps two waves
// per SIMD.
constexpr int kGroupedMaxSlots = 4;

struct ReduceArgs {
  void* out;
  const float* part_o;
  const float* part_lse;
  const int32_t* context_lens;
  int num_seqs;
  int num_heads;
  int max_partitions;
  int partition_tokens;
  int max_context_len;
};

// Next-token sampling, one row of logits per workgroup.
constexpr int kMaxSampleVocab = 32768;   // 32 tokens in registers per thread of 1024
struct SampleArgs {
  const void* logits;      // [num_rows, row_stride], fp32 or bf16
  int64_t row_stride;      // elements between rows
  int vocab;
  int num_rows;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* uniform;    // one draw in [0, 1) per row
  int32_t* tokens;
};

// Pools a batch of whole-block moves reads from and writes to (K and V alike).
struct BlockPools {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  int64_t block_bytes;            // bytes of one physical block of one pool
  int64_t src_blocks;
  int64_t dst_blocks;
  int64_t num_pairs;
};

// Pairs one swap launch carries in its kernel arguments.
constexpr int kSwapPairsPerLaunch = 256;

hipError_t launch_reshape_and_cache(const ScatterArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream);
// Writes a.sched for the dealt split-K decode (one workgroup).
hipError_t launch_decode_schedule(const DecodeArgs& a, hipStream_t stream);
// pa_decode's scalar and pointer checks (no HIP call): PA_OK or the status pa_decode returns.
int check_decode_args(const void* out, const void* query, const void* key_cache,
                      const void* value_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, int max_blocks_per_seq, int64_t num_blocks,
                      int max_context_len, int partition_size, pa_dtype dtype);
// FP8 caches: which (group, head_dim, query type) combinations have a kernel.
bool decode_fp8_supported(int group, int head_dim, bool bf16_query);
hipError_t launch_decode_fp8(const DecodeArgs& a, int head_dim, bool bf16_query,
                             hipStream_t stream);
hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_valu_bf16(const DecodeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_valu_f32(const DecodeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_valu_fp8(const DecodeArgs& a, int head_dim, bool bf16_query,
                                  hipStream_t stream);
hipError_t launch_decode_gqa_mfma_fp8(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_splitk_reduce(const ReduceArgs& a, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_copy_blocks(const BlockPools& pools, const int32_t* block_mapping,
                              hipStream_t stream);
hipError_t launch_swap_blocks(const BlockPools& pools, const int32_t* host_pairs,
                              hipStream_t stream);
hipError_t launch_sample(const SampleArgs& a, bool bf16, hipStream_t stream);

// Stream-read calibration: kStreamBlocks workgroups, one 32-bit fold each (the grid
// and unroll that read fastest in a sweep of 1024..65536 workgroups x unroll 4..16).
constexpr int kStreamBlocks = 32768;
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_prefill_mfma(const DecodeArgs& a, int head_dim, hipStream_t stream);
// The same over FP8 (E4M3) pools; a.scale_log2 includes the K scale, a.v_scale is V's.
hipError_t launch_prefill_mfma_fp8(const DecodeArgs& a, int head_dim, hipStream_t stream);

}  // namespace pa
