// Whole-block copies: copy-on-write inside the pools, and swaps between a
// device pool and a pool in pinned host memory.
//
// When a sequence writes into a partly filled block it still shares with
// others, the block is copied first and the writer continues in the copy
// (intelliparadigm.com article, section 2.2, reference counts for copy on
// write; section 3.3, the block copy itself).  Swap space holds the blocks of
// preempted sequences in host memory (same article, section 5.1).  In the
// [num_blocks, num_kv_heads, block_size, head_dim] pool a physical block is one
// contiguous run of num_kv_heads * block_size * head_dim elements, so every
// move is a plain run of 16-byte pieces, bit for bit.
//
// Work unit: one chunk (kCopyThreads * kCopyUnroll pieces) of one pool (K or V)
// of one pair; a workgroup takes units in a grid-stride loop.  Each thread
// issues all its loads of a chunk before its stores.  The pairs of one call are
// independent (distinct destinations, none of them a source), which is what
// lets every chunk run at once.
//
// Stores are nontemporal: a copied block is read at the earliest by the next
// attention launch, which streams gigabytes past the caches anyway.  Letting
// the stores bypass the caches took the 1024-pair, 13B-shaped copy from 4.9 to
// 5.9 TB/s (read + write), above a plain contiguous device copy of the same
// bytes (5.4 TB/s); nontemporal loads as well were slower (5.1).
//
// Swaps run the same loop with the pairs carried in the kernel arguments (the
// block manager hands them out in host memory), up to kSwapPairsPerLaunch per
// launch: one launch moves a whole batch of scattered blocks over PCIe, where
// one runtime copy per block and pool costs several microseconds each.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 2;
constexpr int64_t kMaxCopyGrid = 1 << 16;   // workgroups; more units are strided over

struct DeviceMapping {                       // pairs in device memory
  const int32_t* pairs;
  __device__ int64_t src(int64_t i) const { return pairs[2 * i]; }
  __device__ int64_t dst(int64_t i) const { return pairs[2 * i + 1]; }
};

struct InlineMapping {                       // pairs in the kernel arguments
  int32_t pairs[2 * kSwapPairsPerLaunch];
  __device__ int64_t src(int64_t i) const { return pairs[2 * i]; }
  __device__ int64_t dst(int64_t i) const { return pairs[2 * i + 1]; }
};

template <typename M>
struct MoveArgs {
  BlockPools pools;
  M map;
};

template <typename U, typename M>
__global__ __launch_bounds__(kCopyThreads) void move_blocks_kernel(MoveArgs<M> a) {
  constexpr int64_t kChunk = (int64_t)kCopyThreads * kCopyUnroll;    // U's per chunk
  const BlockPools& p = a.pools;
  const int64_t block_units = p.block_bytes / (int64_t)sizeof(U);
  const int64_t chunks = (block_units + kChunk - 1) / kChunk;
  const int64_t units = p.num_pairs * 2 * chunks;
  const bool same_pool = p.src_k == p.dst_k;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t pair = u / (2 * chunks);
    const int64_t rest = u - pair * 2 * chunks;
    const int pool = (int)(rest / chunks);
    const int64_t chunk = rest - (int64_t)pool * chunks;
    const int64_t src = a.map.src(pair);
    const int64_t dst = a.map.dst(pair);
    if (src < 0 || src >= p.src_blocks || dst < 0 || dst >= p.dst_blocks) continue;
    if (same_pool && src == dst) continue;
    const U* from = static_cast<const U*>(pool ? p.src_v : p.src_k) + src * block_units +
                    chunk * kChunk;
    U* to = static_cast<U*>(pool ? p.dst_v : p.dst_k) + dst * block_units + chunk * kChunk;
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
      if (e < left) __builtin_nontemporal_store(v[i], to + e);
    }
  }
}

namespace {

template <typename M>
hipError_t launch_moves(const MoveArgs<M>& a, hipStream_t stream) {
  const BlockPools& p = a.pools;
  const auto aligned = [&](uintptr_t m) {
    const uintptr_t bits = reinterpret_cast<uintptr_t>(p.src_k) | reinterpret_cast<uintptr_t>(p.src_v) |
                           reinterpret_cast<uintptr_t>(p.dst_k) | reinterpret_cast<uintptr_t>(p.dst_v) |
                           (uintptr_t)p.block_bytes;
    return (bits & (m - 1)) == 0;
  };
  const auto grid_for = [&](int64_t unit_bytes) {
    const int64_t chunk = unit_bytes * kCopyThreads * kCopyUnroll;
    const int64_t units = p.num_pairs * 2 * ((p.block_bytes + chunk - 1) / chunk);
    return dim3((unsigned)(units < kMaxCopyGrid ? units : kMaxCopyGrid));
  };
  const dim3 block(kCopyThreads);
  if (aligned(16))
    hipLaunchKernelGGL((move_blocks_kernel<u32x4, M>), grid_for(16), block, 0, stream, a);
  else if (aligned(4))
    hipLaunchKernelGGL((move_blocks_kernel<uint32_t, M>), grid_for(4), block, 0, stream, a);
  else
    hipLaunchKernelGGL((move_blocks_kernel<uint16_t, M>), grid_for(2), block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_copy_blocks(const BlockPools& pools, const int32_t* block_mapping,
                              hipStream_t stream) {
  if (pools.num_pairs == 0) return hipSuccess;
  MoveArgs<DeviceMapping> a;
  a.pools = pools;
  a.map.pairs = block_mapping;
  return launch_moves(a, stream);
}

hipError_t launch_swap_blocks(const BlockPools& pools, const int32_t* host_pairs,
                              hipStream_t stream) {
  for (int64_t i = 0; i < pools.num_pairs; i += kSwapPairsPerLaunch) {
    const int64_t n = pools.num_pairs - i < kSwapPairsPerLaunch ? pools.num_pairs - i
                                                                : kSwapPairsPerLaunch;
    MoveArgs<InlineMapping> a;
    a.pools = pools;
    a.pools.num_pairs = n;
    for (int64_t j = 0; j < 2 * n; ++j) a.map.pairs[j] = host_pairs[2 * i + j];
    const hipError_t e = launch_moves(a, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
