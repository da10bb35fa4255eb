// Paged-attention decode entry: kernel choice, plus the split-K merge.
//
// Decode runs on the matrix cores when a grouped-query head group is large
// enough to make q.K^T and p.V dense products (decode_mfma.hip), else on the
// vector ALUs (decode_valu.h).  With split-K, each (sequence, head) leaves one
// normalised partial output and its log-sum-exp per context partition, and
// the merge below combines them: out = sum_p exp(lse_p - M) o_p / sum_p
// exp(lse_p - M) with M = max_p lse_p (exact in real arithmetic).
#include "decode_valu.h"

namespace pa {

// Split-K merge: out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M).
//
// One wave per (sequence, head), four per workgroup.  A first pass takes the
// max of the log-sum-exps with one partition per lane.  Then the wave reads
// four partitions per step: the lanes of quarter q take partition p0 + q and
// 16-byte pieces of its row (D/16 columns a lane), so every step has 2 KB in
// flight per wave (four steps unrolled), and the quarters' sums are added
// across lanes at the end.
constexpr int kReduceWaves = 4;
constexpr int kReduceUnroll = 4;

template <typename T, int D>
__global__ __launch_bounds__(64 * kReduceWaves) void splitk_reduce_kernel(ReduceArgs a) {
  constexpr int E = D / 16;             // columns per lane
  const int row_sh = blockIdx.x * kReduceWaves + wave_uniform(threadIdx.x >> 6);
  if (row_sh >= a.num_seqs * a.num_heads) return;
  const int s = row_sh / a.num_heads;
  const int h = row_sh - s * a.num_heads;
  const int lane = threadIdx.x & (kWave - 1);
  const int len = a.context_lens[s];
  if (len <= 0 || len > a.max_context_len) return;   // the decode kernel wrote these
  const int n = (len + a.partition_tokens - 1) / a.partition_tokens;
  if (n <= 1) return;
  const int64_t row = (int64_t)row_sh * a.max_partitions;
  const float* lse = a.part_lse + row;

  float mm = -INFINITY;
  bool nan = false;
  for (int p0 = 0; p0 < n; p0 += kWave) {
    const float x = p0 + lane < n ? lse[p0 + lane] : -INFINITY;
    nan |= isnan(x);
    mm = fmaxf(mm, x);
  }
  mm = xor_max_above<1>(mm);
  nan = __ballot(nan) != 0;

  const int q = lane >> 4;              // this lane's partition within a step of four
  const int col = (lane & 15) * E;
  float acc[E], wsum = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float* po = a.part_o + row * D + col;
  for (int p0 = 0; p0 < n; p0 += 4 * kReduceUnroll) {
#pragma unroll
    for (int u = 0; u < kReduceUnroll; ++u) {
      const int p = p0 + 4 * u + q;
      if (p < n) {
        const float wt = expf(lse[p] - mm);
        wsum += wt;
        const f32x4* src = reinterpret_cast<const f32x4*>(po + (int64_t)p * D);
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4) {
          const f32x4 v = src[e4];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * e4 + i] = fmaf(wt, v[i], acc[4 * e4 + i]);
        }
      }
    }
  }
  // add the four quarters (lanes l, l ^ 16, l ^ 32, l ^ 48)
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = xor_sum_above<16>(acc[e]);
  wsum = xor_sum_above<16>(wsum);
  if (q == 0) {
    T* dst = static_cast<T*>(a.out) + (int64_t)row_sh * D + col;
#pragma unroll
    for (int e = 0; e < E; ++e)
      dst[e] = ElemTraits<T>::from_f32(nan ? __builtin_nanf("") : acc[e] / wsum);
  }
}

// Schedule of the dealt split-K decode (decode_valu_dealt_kernel).
//
// Order: the (sequence, partition) pairs that have a work unit, sorted by the
// partition's length in blocks, longest first -- a counting sort in one
// workgroup; lengths of kSchedBuckets - 1 blocks and more share the first
// bucket, and pairs of equal length come in any order (the order decides which
// workgroup computes a unit, never its result).  Listed are partition 0 of
// every sequence (which writes the zeros or NaN of a sequence without context
// or with a length outside the contract) and the further partitions of a
// sequence within the contract.  Unit t is kv head t % num_kv_heads of pair
// t / num_kv_heads.
//
// The deal (dealt_unit): the launch hands workgroup b to XCD b % 8, and each
// XCD runs its own workgroups in order of b.  With one unit per workgroup in
// plain order every XCD gets an eighth of the work, but under a full read
// stream the odd-numbered XCDs of this part take about 10% longer per block
// than the even ones (per-workgroup timestamps, also with the kv heads
// rotated across XCDs), so the even ones finish early and idle.  The deal gives
// each even XCD 7 units of every 52 and each odd one 6: of the shares tried
// (1 : 1, 17 : 15, 7 : 6, 17 : 14, 18 : 14) 7 : 6 and 17 : 14 drained the
// Llama-2-13B-shaped batch fastest, about 4% ahead of one workgroup per unit in
// plain order.
constexpr int kSchedThreads = 1024;
constexpr int kSchedBuckets = kSchedThreads;
constexpr int kSchedCached = 4096;   // sequences whose block counts stay in LDS between passes

__device__ __forceinline__ int sched_partitions(const DecodeArgs& a, int s, int& nblk) {
  const int ctx = a.context_lens[s];
  const bool bad = ctx < 0 || ctx > a.max_context_len || ctx > a.max_blocks_per_seq * kBlock;
  nblk = bad ? 0 : (ctx + kBlock - 1) / kBlock;
  const int np = (nblk + a.partition_blocks - 1) / a.partition_blocks;
  return np > 1 ? np : 1;
}

__device__ __forceinline__ int sched_bucket(const DecodeArgs& a, int nblk, int p) {
  const int len = min(nblk - p * a.partition_blocks, a.partition_blocks);
  return kSchedBuckets - 1 - min(len, kSchedBuckets - 1);
}

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(DecodeArgs a) {
  __shared__ int slot[kSchedBuckets];
  __shared__ int wave_total[kSchedThreads / kWave];
  __shared__ int2 cached[kSchedCached];   // (partitions, blocks) of the first sequences
  const int tid = threadIdx.x;
  slot[tid] = 0;
  __syncthreads();
  for (int s = tid; s < a.num_seqs; s += kSchedThreads) {
    int nblk;
    const int np = sched_partitions(a, s, nblk);
    if (s < kSchedCached) cached[s] = make_int2(np, nblk);
    for (int p = 0; p < np; ++p) atomicAdd(&slot[sched_bucket(a, nblk, p)], 1);
  }
  __syncthreads();
  // exclusive prefix sum of the bucket counts: within each wave, then across
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int count = slot[tid];
  int incl = count;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wave_total[w] = incl;
  __syncthreads();
  int before = 0, npairs = 0;
  for (int x = 0; x < kSchedThreads / kWave; ++x) {
    before += x < w ? wave_total[x] : 0;
    npairs += wave_total[x];
  }
  slot[tid] = before + incl - count;   // first position of bucket tid
  if (tid == 0) a.sched[kSchedPairs] = npairs;
  __syncthreads();
  int* const pairs = a.sched + kSchedHeader;
  for (int s = tid; s < a.num_seqs; s += kSchedThreads) {
    int nblk, np;
    if (s < kSchedCached) {
      np = cached[s].x;
      nblk = cached[s].y;
    } else {
      np = sched_partitions(a, s, nblk);
    }
    for (int p = 0; p < np; ++p)
      pairs[atomicAdd(&slot[sched_bucket(a, nblk, p)], 1)] = s * a.max_partitions + p;
  }
}

hipError_t launch_decode_schedule(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
  return hipGetLastError();
}

// Grouped-query decode with at least this many query heads per kv head runs on
// the matrix cores (bf16, head_dim 128); smaller groups stay on the vector ALUs.
constexpr int kMfmaMinGroup = 4;

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  if (bf16 && head_dim == 128 && a.group >= kMfmaMinGroup && a.query_start_loc == nullptr)
    return launch_decode_gqa_mfma(a, stream);
  return bf16 ? launch_decode_valu_bf16(a, head_dim, stream)
              : launch_decode_valu_f32(a, head_dim, stream);
}

// FP8 caches: grouped-query heads (bf16 query, head_dim 128, group >= 4) on the
// matrix cores, the rest on the vector ALUs, whose widened accumulators leave
// room for at most kFp8ValuMaxGroup query heads per kv head.
bool decode_fp8_supported(int group, int head_dim, bool bf16_query) {
  return (bf16_query && head_dim == 128 && group >= kMfmaMinGroup) || group <= kFp8ValuMaxGroup;
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int head_dim, bool bf16_query,
                             hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  if (bf16_query && head_dim == 128 && a.group >= kMfmaMinGroup)
    return launch_decode_gqa_mfma_fp8(a, stream);
  return launch_decode_valu_fp8(a, head_dim, bf16_query, stream);
}

hipError_t launch_splitk_reduce(const ReduceArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
  const dim3 grid((unsigned)((rows + kReduceWaves - 1) / kReduceWaves));
  const dim3 block(64 * kReduceWaves);
  if (bf16) {
    if (head_dim == 64)
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, 64>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, 128>), grid, block, 0, stream, a);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((splitk_reduce_kernel<float, 64>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<float, 128>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
