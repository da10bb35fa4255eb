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

// FP8 (E4M3) caches: the token's fp32 (or bf16-widened) values are multiplied
// by the inverse per-tensor scale, rounded once to fp32, and encoded (nearest,
// ties to even, saturating at 448).  Each thread handles 4 consecutive
// elements of one head row and writes their 4 codes as one word.
template <typename S>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ScatterArgs a) {
  const int64_t tok = blockIdx.x;
  const int64_t slot = a.slot_mapping[tok];
  if (slot < 0 || slot >= a.num_blocks * kBlock) return;
  const int64_t blk = slot / kBlock;
  const int row = (int)(slot % kBlock);
  const int quads = a.head_dim / 4;                    // 4-element groups per head row
  const int total = a.num_kv_heads * quads;
  const S* ksrc = static_cast<const S*>(a.key) + tok * a.key_stride;
  const S* vsrc = static_cast<const S*>(a.value) + tok * a.value_stride;
  uint32_t* kdst = static_cast<uint32_t*>(a.key_cache);
  uint32_t* vdst = static_cast<uint32_t*>(a.value_cache);
  const int64_t base = (blk * a.num_kv_heads * kBlock + row) * (int64_t)quads;
  const auto widen = [](S x) {
    if constexpr (sizeof(S) == 2) return __uint_as_float((uint32_t)x << 16);
    else return x;
  };
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int h = i / quads;
    const int u = i - h * quads;
    const int64_t d = base + (int64_t)h * kBlock * quads + u;
    const S* k = ksrc + 4 * i;
    const S* v = vsrc + 4 * i;
    kdst[d] = f32x4_to_fp8x4(widen(k[0]) * a.k_inv_scale, widen(k[1]) * a.k_inv_scale,
                             widen(k[2]) * a.k_inv_scale, widen(k[3]) * a.k_inv_scale);
    vdst[d] = f32x4_to_fp8x4(widen(v[0]) * a.v_inv_scale, widen(v[1]) * a.v_inv_scale,
                             widen(v[2]) * a.v_inv_scale, widen(v[3]) * a.v_inv_scale);
  }
}

hipError_t launch_reshape_and_cache(const ScatterArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.fp8) {
    const dim3 grid((unsigned)a.num_tokens), block(256);
    if (a.elem_bytes == 4)
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<float>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<bf16_t>, grid, block, 0, stream, a);
    return hipGetLastError();
  }
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
