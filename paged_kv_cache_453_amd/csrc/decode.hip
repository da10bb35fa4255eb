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
// max of the log-sum-exps with one partition per lane; then each lane owns
// D/64 adjacent columns and walks the partitions, the weight of partition p
// broadcast from the lane that computed it.  The partials of successive
// partitions are independent loads, unrolled so that many are in flight --
// the merge is a short stream over the workspace, not a chain of waits.
constexpr int kReduceWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(64 * kReduceWaves) void splitk_reduce_kernel(ReduceArgs a) {
  constexpr int E = D / kWave;          // columns per lane
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

  float acc[E], wsum = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float* po = a.part_o + row * D + lane * E;
  for (int p0 = 0; p0 < n; p0 += kWave) {
    const float wl = p0 + lane < n ? expf(lse[p0 + lane] - mm) : 0.f;
    wsum += wl;
    const int cnt = min(kWave, n - p0);
#pragma unroll 8
    for (int t = 0; t < cnt; ++t) {
      const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), t));
      const float* src = po + (int64_t)(p0 + t) * D;
      if constexpr (E == 2) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        acc[0] = fmaf(wt, v.x, acc[0]);
        acc[1] = fmaf(wt, v.y, acc[1]);
      } else {
        acc[0] = fmaf(wt, src[0], acc[0]);
      }
    }
  }
  wsum = xor_sum_above<1>(wsum);
  T* dst = static_cast<T*>(a.out) + (int64_t)row_sh * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e)
    dst[e] = ElemTraits<T>::from_f32(nan ? __builtin_nanf("") : acc[e] / wsum);
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
