// Stream-read calibration: the HBM read rate this part reaches with plain,
// fully coalesced 16-byte loads, against which the decode kernels (bound by
// HBM reads) are compared.  Not an operation of the method: a measurement aid.
//
// A grid of kStreamBlocks workgroups walks the buffer in grid-stride order,
// each thread keeping kStreamUnroll nontemporal 16-byte loads in flight and
// folding what it reads with XOR; each workgroup stores one 32-bit fold, so
// every byte read reaches a store (and the XOR of the folds is the XOR of the
// buffer's 32-bit words, which a test can check).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 16;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                     int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t fold = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) fold ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    fold ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) fold ^= (uint32_t)__shfl_xor((int)fold, o, 64);
  __shared__ uint32_t wave_fold[kStreamThreads / kWave];
  if ((threadIdx.x & 63) == 0) wave_fold[threadIdx.x >> 6] = fold;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t f = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / kWave; ++w) f ^= wave_fold[w];
    sink[blockIdx.x] = f;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
