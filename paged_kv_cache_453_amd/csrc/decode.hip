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
template <typename T, int D>
__global__ __launch_bounds__(D) void splitk_reduce_kernel(ReduceArgs a) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  const int len = a.context_lens[s];
  if (len <= 0 || len > a.max_context_len) return;   // the decode kernel wrote these
  const int n = (len + a.partition_tokens - 1) / a.partition_tokens;
  if (n <= 1) return;
  const int64_t row = ((int64_t)s * a.num_heads + h) * a.max_partitions;
  const float* lse = a.part_lse + row;
  float mm = -INFINITY;
  bool nan = false;
  for (int p = 0; p < n; ++p) {
    const float x = lse[p];
    nan |= isnan(x);
    mm = fmaxf(mm, x);
  }
  float wsum = 0.f, o = 0.f;
  for (int p = 0; p < n; ++p) {
    const float wgt = expf(lse[p] - mm);
    wsum += wgt;
    o = fmaf(wgt, a.part_o[(row + p) * D + d], o);
  }
  o = nan ? __builtin_nanf("") : o / wsum;
  static_cast<T*>(a.out)[((int64_t)s * a.num_heads + h) * D + d] = ElemTraits<T>::from_f32(o);
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

hipError_t launch_splitk_reduce(const ReduceArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  dim3 grid(a.num_seqs, a.num_heads);
  if (bf16) {
    if (head_dim == 64)
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, 64>), grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, 128>), grid, dim3(128), 0, stream, a);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((splitk_reduce_kernel<float, 64>), grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<float, 128>), grid, dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
