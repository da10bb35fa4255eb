// Next-token sampling: temperature, top-k, top-p and the draw, fused in one
// kernel with no sort ("vLLM 基本原理", section FlashInfer 采样器: the model's
// logits are scaled by the temperature, top-k keeps the K most probable
// tokens, top-p the most probable ones whose cumulative probability reaches P,
// and the next token is drawn from what is left; a fused sampler avoids
// sorting the logits and is statistically equivalent to the plain one).
//
// One workgroup (1024 threads) per row.  The row's scaled logits z = x / T
// are staged once from HBM into LDS (padded one word per 32 so that each
// thread's contiguous chunk is read without bank conflicts); every later pass
// reads LDS.
//  - Order keys: z's fp32 bits mapped to uint32 so that key order is z order
//    (NaN counts as -inf).
//  - Top-k: the K-th largest key by a 4-pass radix select over 8-bit digits,
//    with exact integer counts in an LDS histogram; tokens tied with it stay.
//  - Weights: w = exp(z - max z) in fixed point (40 fraction bits) as 64-bit
//    integers, so every sum is exact and independent of the summation order.
//  - Top-p: the largest key t whose mass {key >= t} reaches P times the top-k
//    mass, by the same radix select with 64-bit mass histograms.  Every token
//    at or above it is one whose strictly-more-probable mass is below P.
//  - Draw: an exclusive scan of the per-thread chunk masses (in vocabulary
//    order) locates floor(u * total); the owning thread walks its chunk to
//    the token, the inverse of the distribution function.
// Per-row parameters that are out of range (T <= 0, P outside (0, 1], u
// outside [0, 1)) and rows with no finite logit give token -1; +inf logits
// share all the probability.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr float kWeightScale = 1099511627776.f;   // 2^40

__device__ __forceinline__ int lds_index(int i) { return i + (i >> 5); }

__device__ __forceinline__ float logit_f32(float x) { return x; }
__device__ __forceinline__ float logit_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t b = __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t weight_of(float z, float m) {
  const float e = __builtin_amdgcn_exp2f((z - m) * kLog2e);   // in [0, 1]
  return (uint64_t)(e * kWeightScale);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t x, int d) {
  const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)x, d, 64);
  const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(x >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t x, int d) {
  const uint32_t lo = (uint32_t)__shfl_down((int)(uint32_t)x, d, 64);
  const uint32_t hi = (uint32_t)__shfl_down((int)(uint32_t)(x >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

struct SampleShared {
  float z[kMaxSampleVocab + kMaxSampleVocab / 32];
  uint64_t bins[256];
  uint64_t wave_part[kSampleWaves];
  float wave_max[kSampleWaves];
  uint64_t sel_above;
  uint32_t sel_prefix;
  int token;
};

// Sum of a uint64 over the workgroup, the same in every thread.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t x, SampleShared& sh) {
  for (int o = 32; o > 0; o >>= 1) x += shfl_xor_u64(x, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.wave_part[w] = x;
  __syncthreads();
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < kSampleWaves; ++i) s += sh.wave_part[i];
  return s;
}

// Radix select over the keys of this thread's chunk: the largest key t with
// amount{key >= t} >= target, where a token's amount is 1 (COUNT) or its
// weight, and only tokens with key >= floor_key take part.
template <bool COUNT>
__device__ uint32_t radix_select(SampleShared& sh, int i0, int i1, float m, uint32_t floor_key,
                                 uint64_t target) {
  uint32_t prefix = 0;
  uint64_t above = 0;   // amount of the tokens whose key is above the current prefix range
  for (int level = 0; level < 4; ++level) {
    const int shift = 24 - 8 * level;
    if (threadIdx.x < 256) sh.bins[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t hi_mask = level == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = i0; i < i1; ++i) {
      const float z = sh.z[lds_index(i)];
      const uint32_t k = order_key(z);
      if (k < floor_key || (k & hi_mask) != (prefix & hi_mask)) continue;
      const uint64_t amount = COUNT ? 1u : weight_of(z, m);
      if (amount) atomicAdd(reinterpret_cast<unsigned long long*>(&sh.bins[(k >> shift) & 255]),
                            (unsigned long long)amount);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
      const int l = threadIdx.x;
      const uint64_t b0 = sh.bins[4 * l], b1 = sh.bins[4 * l + 1], b2 = sh.bins[4 * l + 2],
                     b3 = sh.bins[4 * l + 3];
      const uint64_t mine = b0 + b1 + b2 + b3;
      uint64_t suffix = mine;   // sum over lanes >= l
      for (int d = 1; d < 64; d <<= 1) {
        const uint64_t o = shfl_down_u64(suffix, d);
        if (l + d < 64) suffix += o;
      }
      const uint64_t higher = suffix - mine;   // lanes > l
      // the chosen lane is the highest one whose suffix reaches the target
      const bool reach = above + suffix >= target;
      const uint64_t ballot = __ballot(reach);
      const int chosen = ballot ? 63 - __builtin_clzll(ballot) : 0;
      if (l == chosen) {
        uint64_t acc = above + higher;
        int digit = 4 * l;
        const uint64_t b[4] = {b0, b1, b2, b3};
        for (int j = 3; j >= 0; --j) {
          if (acc + b[j] >= target) {
            digit = 4 * l + j;
            break;
          }
          acc += b[j];
        }
        sh.sel_prefix = prefix | ((uint32_t)digit << shift);
        sh.sel_above = acc;
      }
    }
    __syncthreads();
    prefix = sh.sel_prefix;
    above = sh.sel_above;
  }
  return prefix;
}

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleArgs a) {
  __shared__ SampleShared sh;
  const int row = blockIdx.x;
  const int V = a.vocab;
  const float temp = a.temperature[row];
  const int top_k = a.top_k[row];
  const float top_p = a.top_p[row];
  const float u = a.uniform[row];
  if (!(temp > 0.f) || !(top_p > 0.f && top_p <= 1.f) || !(u >= 0.f && u < 1.f)) {
    if (threadIdx.x == 0) a.tokens[row] = -1;
    return;
  }
  const float inv_t = 1.f / temp;

  // stage z = x / T into LDS (coalesced reads), and the row max
  const T* x = static_cast<const T*>(a.logits) + (int64_t)row * a.row_stride;
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < V; i += kSampleThreads) {
    float z = logit_f32(x[i]) * inv_t;
    z = isnan(z) ? -INFINITY : fminf(z, 3.402823466e38f);   // +inf: the largest finite value
    sh.z[lds_index(i)] = z;
    mx = fmaxf(mx, z);
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) sh.wave_max[threadIdx.x >> 6] = mx;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSampleWaves; ++i) m = fmaxf(m, sh.wave_max[i]);
  if (m == -INFINITY) {
    if (threadIdx.x == 0) a.tokens[row] = -1;
    return;
  }

  const int chunk = (V + kSampleThreads - 1) / kSampleThreads;
  const int i0 = min(V, (int)threadIdx.x * chunk);
  const int i1 = min(V, i0 + chunk);
  const uint32_t live_key = order_key(-INFINITY) + 1;   // finite or +inf

  uint32_t thr = live_key;
  if (top_k > 0 && top_k < V) thr = radix_select<true>(sh, i0, i1, m, live_key, (uint64_t)top_k);

  const auto chunk_mass = [&](uint32_t t) {
    uint64_t s = 0;
    for (int i = i0; i < i1; ++i) {
      const float z = sh.z[lds_index(i)];
      if (order_key(z) >= t) s += weight_of(z, m);
    }
    return s;
  };
  if (top_p < 1.f) {
    const uint64_t zk = block_sum_u64(chunk_mass(thr), sh);
    const uint64_t target = (uint64_t)ceil((double)top_p * (double)zk);
    thr = radix_select<false>(sh, i0, i1, m, thr, target > 0 ? target : 1);
  }

  // the draw: exclusive scan of the chunk masses in vocabulary order
  const uint64_t mine = chunk_mass(thr);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t incl = mine;
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up_u64(incl, d);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) sh.wave_part[w] = incl;
  if (threadIdx.x == 0) sh.token = -1;
  __syncthreads();
  uint64_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kSampleWaves; ++i) {
    before += i < w ? sh.wave_part[i] : 0;
    total += sh.wave_part[i];
  }
  const uint64_t excl = before + incl - mine;
  uint64_t target = (uint64_t)((double)u * (double)total);
  target = target < total ? target : total - 1;   // u < 1, whatever the double rounding
  if (mine > 0 && excl <= target && target < excl + mine) {
    uint64_t acc = excl;
    for (int i = i0; i < i1; ++i) {
      const float z = sh.z[lds_index(i)];
      if (order_key(z) < thr) continue;
      acc += weight_of(z, m);
      if (acc > target) {
        sh.token = i;
        break;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.tokens[row] = sh.token;
}

hipError_t launch_sample(const SampleArgs& a, bool bf16, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_rows), block(kSampleThreads);
  if (bf16)
    hipLaunchKernelGGL(sample_kernel<bf16_t>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(sample_kernel<float>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
