// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kBlock = 16;          // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint16_t bf16_t;            // bf16 kept as its bit pattern in memory
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 <-> fp32 -------------------------------------------------------
// A bf16 value is the top half of an fp32 word, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Reinterpret one 32-bit word as two bf16 lanes.  Takes the word by value:
// bit-casting a vector element expression in place (vec[i]) has been seen to
// read element 0 whatever i is, so callers pass a plain scalar.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(bf16_t, b);
}
// Two fp32 -> bf16 (nearest even) in one v_cvt_pk_bf16_f32; lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// ---- fp8 (OCP E4M3) <-> fp32 ------------------------------------------------
// An E4M3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
// infinities, NaN = S.1111.111, largest magnitude 448) kept as its byte.
typedef uint8_t fp8_t;
constexpr float kFp8Max = 448.f;

// Four codes of one word (byte i = element i) -> four fp32 values, exact; the
// gfx950 conversion reads the OCP E4M3 format.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = hi.x;
  out[3] = hi.y;
}

// Four codes -> four bf16 (two words, element 0 in the low half of word 0).
// Exact: every E4M3 value has at most 4 significant bits.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  float f[4];
  fp8x4_to_f32(w, f);
  return u32x2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
}

// Four fp32 values -> four codes (element i in byte i): nearest, ties to even
// (the hardware conversion), after saturating magnitudes above 448 to 448 (the
// hardware would give NaN there); NaN gives 0x7F.
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  const auto sat = [](float x) { return fminf(fmaxf(x, -kFp8Max), kFp8Max); };
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), (int)w, true);
  const float x[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (isnan(x[i])) w = (w & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i));
  return w;
}

// ---- cross-lane sums inside groups of 2/4/8/16 lanes (DPP, no LDS) --------
// quad_perm [1,0,3,2] swaps neighbours, [2,3,0,1] swaps pairs, half-row mirror
// maps lane i of an 8-lane half onto 7-i, row mirror maps lane i of a 16-lane
// row onto 15-i.  After the quad steps every lane of a quad holds the quad sum,
// so each mirror step adds the partner quad / half and the sums stay exact
// group totals in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  if constexpr (N >= 2) x += dpp_f32<0xB1>(x);     // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_f32<0x4E>(x);     // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_f32<0x141>(x);    // row_half_mirror
  if constexpr (N >= 16) x += dpp_f32<0x140>(x);   // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// max over lanes that differ only in the lane-index bits [LO, 64): a
// butterfly with shuffles (used once per workgroup, off the hot loop).
template <int LO>
__device__ __forceinline__ float xor_max_above(float x) {
#pragma unroll
  for (int o = LO; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
template <int LO>
__device__ __forceinline__ float xor_sum_above(float x) {
#pragma unroll
  for (int o = LO; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Workgroup barrier that orders LDS only.  __syncthreads() also releases global
// memory, which makes every wave wait for all of its outstanding global loads
// (vmcnt 0) at the barrier; a kernel that prefetches the next tile from global
// memory while computing on LDS must not pay that.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace pa
