// reshape_and_cache: copy each new token's K and V rows into its cache slot.
//
// The cache keeps every token's K/V so later tokens attend to it without
// recomputation ("vLLM 基本原理", section "什么是 KV Cache"); the slot of a token
// names a physical block and a row inside it, the pool being laid out as
// [num_blocks, num_kv_heads, block_size, head_dim] (intelliparadigm.com
// article, section 3.1).  Pure data movement: the copy is bit-exact.
//
// One workgroup per token.  Threads walk the token's num_kv_heads * head_dim
// elements in 16-byte pieces when every address and stride allows it, else in
// whole elements.  Source rows of a token are contiguous; destination rows for
// different heads sit block_size rows apart.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <typename U>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ScatterArgs a) {
  const int64_t tok = blockIdx.x;
  const int64_t slot = a.slot_mapping[tok];
  if (slot < 0 || slot >= a.num_blocks * kBlock) return;
  const int64_t blk = slot / kBlock;
  const int row = (int)(slot % kBlock);
  const int per_elem = (int)sizeof(U) / a.elem_bytes;      // elements in one U
  const int row_units = a.head_dim / per_elem;             // U's per head row
  const int total = a.num_kv_heads * row_units;
  const U* ksrc = reinterpret_cast<const U*>(static_cast<const char*>(a.key) +
                                             tok * a.key_stride * a.elem_bytes);
  const U* vsrc = reinterpret_cast<const U*>(static_cast<const char*>(a.value) +
                                             tok * a.value_stride * a.elem_bytes);
  U* kdst = static_cast<U*>(a.key_cache);
  U* vdst = static_cast<U*>(a.value_cache);
  const int64_t base = (blk * a.num_kv_heads * kBlock + row) * (int64_t)row_units;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int h = i / row_units;
    const int u = i - h * row_units;
    const int64_t d = base + (int64_t)h * kBlock * row_units + u;
    kdst[d] = ksrc[i];
    vdst[d] = vsrc[i];
  }
}

hipError_t launch_reshape_and_cache(const ScatterArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = aligned16(a.key) && aligned16(a.value) && aligned16(a.key_cache) &&
                   aligned16(a.value_cache) && (a.key_stride * a.elem_bytes) % 16 == 0 &&
                   (a.value_stride * a.elem_bytes) % 16 == 0 && (a.head_dim * a.elem_bytes) % 16 == 0;
  dim3 grid((unsigned)a.num_tokens), block(256);
  if (vec) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<u32x4>, grid, block, 0, stream, a);
  } else if (a.elem_bytes == 4) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint32_t>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint16_t>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
