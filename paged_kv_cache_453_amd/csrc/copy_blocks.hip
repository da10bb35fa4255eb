// copy_blocks: copy whole physical blocks inside the K and V pools.
//
// When a sequence writes into a partly filled block it still shares with
// others, the block is copied first and the writer continues in the copy
// (intelliparadigm.com article, section 2.2, reference counts for copy on
// write; section 3.3, the block copy itself).  In the
// [num_blocks, num_kv_heads, block_size, head_dim] pool a physical block is one
// contiguous run of num_kv_heads * block_size * head_dim elements, so a copy is
// a plain run of 16-byte moves, bit for bit.
//
// Work unit: one chunk of kChunkBytes of one pool of one pair; a workgroup takes
// units in a grid-stride loop.  Each thread issues all its loads of a chunk
// before its stores, so a wave keeps kUnroll 16-byte loads in flight.  The pairs
// of one call are independent (distinct destinations, none of them a source),
// which is what lets every chunk run at once.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kMaxCopyGrid = 1 << 16;   // workgroups; more units are strided over

template <typename U>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a) {
  constexpr int64_t kChunk = (int64_t)kCopyThreads * kCopyUnroll;    // U's per chunk
  const int64_t block_units = a.block_bytes / (int64_t)sizeof(U);
  const int64_t chunks = (block_units + kChunk - 1) / kChunk;
  const int64_t units = a.num_pairs * 2 * chunks;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t pair = u / (2 * chunks);
    const int64_t rest = u - pair * 2 * chunks;
    const int pool = (int)(rest / chunks);
    const int64_t chunk = rest - (int64_t)pool * chunks;
    const int64_t src = a.block_mapping[2 * pair];
    const int64_t dst = a.block_mapping[2 * pair + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) continue;
    U* base = static_cast<U*>(pool ? a.value_cache : a.key_cache);
    const U* from = base + src * block_units + chunk * kChunk;
    U* to = base + dst * block_units + chunk * kChunk;
    const int64_t left = block_units - chunk * kChunk;
    U v[kCopyUnroll];
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int64_t e = (int64_t)i * kCopyThreads + threadIdx.x;
      if (e < left) v[i] = from[e];
    }
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int64_t e = (int64_t)i * kCopyThreads + threadIdx.x;
      if (e < left) to[e] = v[i];
    }
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  const auto aligned = [&](uintptr_t m) {
    return ((reinterpret_cast<uintptr_t>(a.key_cache) | reinterpret_cast<uintptr_t>(a.value_cache) |
             (uintptr_t)a.block_bytes) & (m - 1)) == 0;
  };
  const auto grid_for = [&](int64_t unit_bytes) {
    const int64_t chunk = unit_bytes * kCopyThreads * kCopyUnroll;
    const int64_t units = a.num_pairs * 2 * ((a.block_bytes + chunk - 1) / chunk);
    return dim3((unsigned)(units < kMaxCopyGrid ? units : kMaxCopyGrid));
  };
  const dim3 block(kCopyThreads);
  if (aligned(16))
    hipLaunchKernelGGL(copy_blocks_kernel<u32x4>, grid_for(16), block, 0, stream, a);
  else if (aligned(4))
    hipLaunchKernelGGL(copy_blocks_kernel<uint32_t>, grid_for(4), block, 0, stream, a);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<uint16_t>, grid_for(2), block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
