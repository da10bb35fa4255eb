// Next-token sampling: temperature, top-k, top-p and the draw, fused in one
// kernel with no sort ("vLLM 基本原理", section FlashInfer 采样器: the model's
// logits are scaled by the temperature, top-k keeps the K most probable
// tokens, top-p the most probable ones whose cumulative probability reaches P,
// and the next token is drawn from what is left; a fused sampler avoids
// sorting the logits and is statistically equivalent to the plain one).
//
// One workgroup (1024 threads) per row; the row stays in registers for the
// whole kernel (C = 1, 2, 4, ..., 32 tokens a thread, the least that covers
// it), so every pass over it is an unrolled loop of register arithmetic and
// LDS holds only histograms and workgroup partials.  Wave w owns the span
// [64*C*w, 64*C*(w+1)), which it reads in rows of 64 coalesced 16-byte loads:
// lane l holds the G-token group at 64*G*r + G*l of the span in row r.
//  - Weights: f = min(exp(z - max z) * 2^32, 2^32 - 256) in fp32 (the scaling
//    is exact), z = x / T, and the weight w = floor(f), a 32-bit integer; sums
//    of weights are 64-bit, exact and independent of the summation order.  A
//    token more than 2^32 times less likely than the most likely one has
//    weight 0 and takes no part.
//  - Ranks: for f >= 1, the bits of f less those of 1.0 -- a 28-bit integer
//    (5 bits of octave, 23 of mantissa) that orders like z, from which w is
//    recovered exactly; this is what the registers hold.  Tokens tie when
//    their f are equal.
//  - Top-k: the K-th largest rank by a radix select with exact integer
//    counts: a first digit of 8 bits (an eighth of an octave a bucket) over
//    the whole row, with one LDS histogram per lane of a half-wave so that an
//    atomic instruction's lanes never meet on an address; then the tokens of
//    the chosen bucket are gathered into LDS (a slice per wave, positions
//    from the wave's ballot) and the remaining digits (8, 8, 4 bits) are
//    resolved over them alone, in one small histogram per level (over the row
//    again if a slice overflows).  Tokens tied with the K-th stay.  The select
//    stops at the first digit whose bucket closes the count exactly.
//  - Top-p: the largest rank t whose mass {rank >= t} reaches P times the
//    top-k mass, by the same select with 64-bit mass histograms; the top-k
//    mass is the total of its first histogram.  Every token at or above it is
//    one whose strictly-more-probable mass is below P.  When a top-p follows
//    a top-k whose bucket and everything above it are at most kGatherAll
//    tokens, the top-k gather takes all of them, and the top-p select then
//    runs over the list alone.
//  - Draw: a scan of the wave masses (from the list when it holds every kept
//    token, else from the registers) locates floor(u * total) in a wave; that
//    wave scans its rows (DPP lane moves) to the lane whose group holds it,
//    and the lane walks the group to the token: the inverse of the
//    distribution function.
// Per-row parameters that are out of range (T <= 0, P outside (0, 1], u
// outside [0, 1)) and rows with no finite logit give token -1; +inf logits
// share all the probability.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kLaneCopies = 32;     // histogram copies, one per lane of a half-wave
constexpr int kSlice = 512;         // a wave's share of the LDS list of gathered tokens
constexpr int kGatherAll = 6144;    // gather all tokens above a bucket up to this many
constexpr int kRankBits = 28;
constexpr uint32_t kRankEnd = 1u << kRankBits;
constexpr uint32_t kKeyOne = 0x3F800000u;   // fp32 bits of 1.0
static_assert(kMaxSampleVocab <= 32 * kSampleThreads, "a thread holds at most 32 tokens");

__device__ __forceinline__ float logit_f32(float x) { return x; }
__device__ __forceinline__ float logit_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

constexpr uint32_t kNoRank = 0xFFFFFFFFu;   // weight 0: takes part in nothing

// Rank of a token from e = exp(z - max z), and the weight it stands for.
__device__ __forceinline__ uint32_t rank_of_e(float e) {
  const float f = fminf(e * 4294967296.f, 4294967040.f);
  return f >= 1.f ? __float_as_uint(f) - kKeyOne : kNoRank;
}
__device__ __forceinline__ uint32_t weight_of(uint32_t rk) {   // 0 for kNoRank
  return (uint32_t)__uint_as_float(rk + kKeyOne);
}
// rank >= floor for a token of weight >= 1, in one unsigned compare
__device__ __forceinline__ bool ranked_at_least(uint32_t rk, uint32_t floor) {
  return rk - floor < kRankEnd - floor;
}

// Keeps the compiler from hoisting per-token ranks out of the passes over the
// row (32 more live registers per thread): each pass recomputes them.
template <int C>
__device__ __forceinline__ void fence_row(uint32_t (&v)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) asm volatile("" : "+v"(v[c]));
}

// ---- wave-wide scans on DPP lane moves (row shifts within 16 lanes, then
// broadcasts of lanes 15 and 31 across rows) --------------------------------
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {   // 0 where no source lane
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t add_dpp(uint64_t v) {
  const uint32_t lo = dpp0<CTRL, ROWS>((uint32_t)v);
  const uint32_t hi = dpp0<CTRL, ROWS>((uint32_t)(v >> 32));
  return v + (((uint64_t)hi << 32) | lo);
}
// inclusive prefix sum over the lanes of the wave
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  v = add_dpp<0x111, 0xF>(v);   // row_shr:1
  v = add_dpp<0x112, 0xF>(v);   // row_shr:2
  v = add_dpp<0x114, 0xF>(v);   // row_shr:4
  v = add_dpp<0x118, 0xF>(v);   // row_shr:8
  v = add_dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = add_dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float max_dpp(float x) {   // x itself where no source lane
  const float o = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROWS, 0xF, false));
  return fmaxf(x, o);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = max_dpp<0x111, 0xF>(v);
  v = max_dpp<0x112, 0xF>(v);
  v = max_dpp<0x114, 0xF>(v);
  v = max_dpp<0x118, 0xF>(v);
  v = max_dpp<0x142, 0xA>(v);
  v = max_dpp<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// sum over each aligned group of four lanes (quad permutes [1,0,3,2], [2,3,0,1])
template <int CTRL>
__device__ __forceinline__ uint64_t quad_dpp(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t quad_sum_u64(uint64_t v) {
  v += quad_dpp<0xB1>(v);
  v += quad_dpp<0x4E>(v);
  return v;
}

struct SampleShared {
  union {
    // one histogram per lane of a half-wave, [bin][copy]: 64-bit masses or
    // 32-bit counts
    uint64_t mass[256][kLaneCopies];
    uint32_t count[256][kLaneCopies];
    } hist;
  uint32_t list[kSampleWaves][kSlice];     // gathered tokens' ranks, a slice per wave
  // a level's bin totals; three in rotation, so that a level over the list
  // needs two barriers: level L fills bins[L % 3] while bins[(L + 2) % 3] is
  // cleared
  uint64_t bins[3][256];
  uint64_t wave_part[kSampleWaves];
  float wave_max[kSampleWaves];
  int slice_n[kSampleWaves];
  uint64_t sel_above;
  uint64_t sel_ge;      // amount at or above the chosen bucket's lower bound
  uint64_t sel_target;
  uint32_t sel_prefix;
  int sel_done;
  int token;
};

// Where a select leaves its answer: the rank floor, and whether the LDS list
// holds every token at or above it.
struct Selected {
  uint32_t floor;
  bool listed;
};

// Radix select over the ranks of the row: the largest rank t with
// amount{rank >= t} >= target, where a token's amount is 1 (COUNT) or its
// weight, and only tokens with weight >= 1 and rank >= floor take part.  In
// mass mode the target is ceil(frac * total amount), at least 1.  Every token
// taking part has an amount of at least 1, so a bucket that brings the amount
// above it to exactly the target holds no token below the answer: the select
// stops there and returns the bucket's lower bound, which keeps the same
// tokens.  If fewer than the target take part, all of them are kept (floor).
//
// With `from_list` the list already holds every token taking part and all
// four digits are resolved over it.  Otherwise the first digit is counted
// over the row, and then every token at or above the chosen bucket is
// gathered into the list; if a wave's slice overflows, the remaining digits
// go over the row again.
template <bool COUNT, int C>
__device__ Selected radix_select(SampleShared& sh, uint32_t (&rank)[C], uint32_t floor,
                                 uint64_t target, double frac, bool from_list, bool cover) {
  constexpr int kWords = COUNT ? 256 * kLaneCopies : 2 * 256 * kLaneCopies;   // 32-bit words
  const int copy = threadIdx.x % kLaneCopies;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t prefix = 0;
  uint64_t above = 0;       // amount of the tokens whose rank is above the current prefix range
  bool listed = from_list;  // the list holds every token taking part in this level
  bool covers = from_list;  // the list holds every token at or above the answer
  const int n_own = sh.slice_n[wv];   // meaningful once listed
  int n_list = n_own;
  // (a previous select read its bins before its last barrier)
  if (threadIdx.x < 512) (&sh.bins[0][0])[threadIdx.x] = 0;   // bins[0] and bins[1]
  for (int level = 0; level < 4; ++level) {
    // digits: bits 27..20, 19..12, 11..4, 3..0
    const int shift = level < 3 ? 20 - 8 * level : 0;
    const uint32_t dmask = level < 3 ? 255u : 15u;
    const int hi_shift = level == 0 ? kRankBits : shift + (level < 3 ? 8 : 4);
    const uint32_t want_hi = prefix >> hi_shift;   // 0 at level 0
    uint64_t* bins = sh.bins[level % 3];
    if (listed) {
      // the gathered tokens: one plain histogram
      if (level == 0) __syncthreads();   // bins cleared
      for (int i = lane; i < n_list; i += 64) {
        const uint32_t rk = sh.list[wv][i];
        if ((rk >> hi_shift) == want_hi && rk >= floor)
          atomicAdd(reinterpret_cast<unsigned long long*>(&bins[(rk >> shift) & dmask]),
                    (unsigned long long)(COUNT ? 1u : weight_of(rk)));
      }
      __syncthreads();
    } else {
      {
        u32x4* h = reinterpret_cast<u32x4*>(&sh.hist);
        for (int i = threadIdx.x; i < kWords / 4; i += kSampleThreads) h[i] = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
      fence_row(rank);
      if (level == 0) {
        // nearly every token takes part: no branches, an amount of 0 for the rest
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const uint32_t rk = rank[c];
          const bool in = ranked_at_least(rk, floor);
          const int d = (rk >> shift) & 255;
          if (COUNT)
            atomicAdd(&sh.hist.count[d][copy], in ? 1u : 0u);
          else
            atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hist.mass[d][copy]),
                      (unsigned long long)(in ? weight_of(rk) : 0u));
        }
      } else {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const uint32_t rk = rank[c];
          if ((rk >> hi_shift) == want_hi && rk >= floor) {
            const int d = (rk >> shift) & dmask;
            if (COUNT)
              atomicAdd(&sh.hist.count[d][copy], 1u);
            else
              atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hist.mass[d][copy]),
                        (unsigned long long)weight_of(rk));
          }
        }
      }
      __syncthreads();
      // four threads a bin, eight copies each, visited in a rotated order so
      // that the lanes of a read fall on distinct banks
      const int b = threadIdx.x >> 2, q = (threadIdx.x & 3) * (kLaneCopies / 4);
      uint64_t t = 0;
#pragma unroll
      for (int j = 0; j < kLaneCopies / 4; ++j) {
        const int cp = q + ((j + b) & (kLaneCopies / 4 - 1));
        t += COUNT ? (uint64_t)sh.hist.count[b][cp] : sh.hist.mass[b][cp];
      }
      t = quad_sum_u64(t);
      if ((threadIdx.x & 3) == 0) bins[b] = t;
      __syncthreads();
    }
    if (threadIdx.x >= 64 && threadIdx.x < 64 + 256)
      sh.bins[(level + 2) % 3][threadIdx.x - 64] = 0;   // for level + 2, while wave 0 scans
    if (threadIdx.x < 64) {
      // lane l holds bins 4l .. 4l+3; the amount in bins above 4l+3 is the
      // total less the inclusive prefix
      const int l = threadIdx.x;
      const uint64_t b0 = bins[4 * l], b1 = bins[4 * l + 1], b2 = bins[4 * l + 2],
                     b3 = bins[4 * l + 3];
      const uint64_t mine = b0 + b1 + b2 + b3;
      const uint64_t incl = wave_scan_u64(mine);
      const uint64_t total = lane_u64(incl, 63);
      const uint64_t higher = total - incl;    // lanes > l
      const uint64_t suffix = higher + mine;   // lanes >= l
      if (level == 0 && frac > 0.0) {
        const uint64_t t = (uint64_t)ceil(frac * (double)total);
        target = t > 0 ? t : 1;
      }
      // the chosen lane is the highest one whose suffix reaches the target
      const bool reach = above + suffix >= target;
      const uint64_t ballot = __ballot(reach);
      const int chosen = ballot ? 63 - __builtin_clzll(ballot) : 0;
      if (!ballot) {
        if (l == 0) {
          sh.sel_prefix = floor;
          sh.sel_above = above;
          sh.sel_ge = above + suffix;
          sh.sel_target = target;
          sh.sel_done = 1;
        }
      } else if (l == chosen) {
        uint64_t acc = above + higher;
        int digit = 4 * l;
        uint64_t ge = acc;
        const uint64_t bk[4] = {b0, b1, b2, b3};
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (ge < target) {   // not reached yet: bin j is the next candidate
            digit = 4 * l + j;
            acc = ge;
            ge += bk[j];
          }
        }
        const bool exact = ge == target;
        sh.sel_prefix = prefix | ((uint32_t)digit << shift);
        sh.sel_above = acc;
        sh.sel_ge = ge;
        sh.sel_target = target;
        sh.sel_done = exact;
      }
    }
    __syncthreads();
    prefix = sh.sel_prefix;
    above = sh.sel_above;
    target = sh.sel_target;
    if (level == 0 && !listed) {
      // Gather into this wave's slice of the list (lane positions from the
      // wave's ballot, no atomics) the tokens the later levels need: with
      // `cover`, and when the count says they are few, every token at or
      // above the chosen bucket, so that a later select over the same tokens
      // and the draw can work from the list too; otherwise the chosen bucket.
      fence_row(rank);
      const bool all_above = COUNT && cover && sh.sel_ge <= (uint64_t)kGatherAll;
      const uint32_t low = max(prefix, floor);
      const uint32_t bucket = prefix >> shift;
      int n = 0;   // wave-uniform
      const auto put = [&](int c, bool member) {
        const uint64_t bl = __ballot(member);
        if (bl) {
          const int pos = n + (int)__builtin_amdgcn_mbcnt_hi(
                                  (uint32_t)(bl >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bl, 0u));
          if (member && pos < kSlice) sh.list[wv][pos] = rank[c];
          n += __popcll(bl);
        }
      };
      if (all_above) {
#pragma unroll
        for (int c = 0; c < C; ++c) put(c, ranked_at_least(rank[c], low));
      } else {
#pragma unroll
        for (int c = 0; c < C; ++c) put(c, (rank[c] >> shift) == bucket && rank[c] >= floor);
      }
      if (lane == 0) sh.slice_n[wv] = n;
      __syncthreads();
      bool fits = true;
#pragma unroll
      for (int i = 0; i < kSampleWaves; ++i) fits = fits && sh.slice_n[i] <= kSlice;
      listed = fits;
      covers = fits && all_above;
      n_list = n;
    }
    if (sh.sel_done) break;
  }
  return Selected{prefix, covers};
}

template <typename T, int C>
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

  // Token of register slot c: group c / G, position c % G in it.
  constexpr int kVec = 16 / (int)sizeof(T);   // tokens in a 16-byte load
  constexpr int G = C < kVec ? C : kVec;      // tokens a lane holds contiguously
  constexpr int R = C / G;                    // rows a wave reads
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int span = wv * 64 * C;
  const auto token_of = [&](int c) { return span + (c / G) * 64 * G + lane * G + c % G; };

  // z = x / T (NaN and the tail past V: -inf)
  const T* x = static_cast<const T*>(a.logits) + (int64_t)row * a.row_stride;
  float z[C];
  if constexpr (G == kVec) {
    const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = token_of(r * G);
      if (vec && i + G <= V) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(x + i);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (sizeof(T) == 4) {
            z[r * G + c] = __uint_as_float(q[c]);
          } else {
            z[r * G + 2 * c] = bf16_lo(q[c]);
            z[r * G + 2 * c + 1] = bf16_hi(q[c]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < G; ++c) z[r * G + c] = i + c < V ? logit_f32(x[i + c]) : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = token_of(c);
      z[c] = i < V ? logit_f32(x[i]) : -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float v = z[c] * inv_t;
    v = isnan(v) ? -INFINITY : fminf(v, 3.402823466e38f);   // +inf: the largest finite value
    z[c] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max_f32(mx);
  if (lane == 0) sh.wave_max[wv] = mx;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSampleWaves; ++i) m = fmaxf(m, sh.wave_max[i]);
  if (m == -INFINITY) {
    if (threadIdx.x == 0) a.tokens[row] = -1;
    return;
  }

  uint32_t rank[C];
#pragma unroll
  for (int c = 0; c < C; ++c) rank[c] = rank_of_e(__builtin_amdgcn_exp2f((z[c] - m) * kLog2e));

  Selected sel{0u, false};   // rank floor 0: every token with weight >= 1
  if (top_k > 0 && top_k < V)
    sel = radix_select<true>(sh, rank, 0u, (uint64_t)top_k, 0.0, false, top_p < 1.f);
  if (top_p < 1.f) sel = radix_select<false>(sh, rank, sel.floor, 1, (double)top_p, sel.listed, false);
  const uint32_t thr = sel.floor;

  // The draw: floor(u * total) located in vocabulary order -- the wave by a
  // scan of the wave masses, then in that wave the row and lane by a scan of
  // each row's group masses, then the token by the lane's walk of its group.
  const auto kept = [&](int c) -> uint32_t {
    return ranked_at_least(rank[c], thr) ? weight_of(rank[c]) : 0u;
  };
  uint64_t mine = 0;
  if (sel.listed) {
    // every kept token is in this wave's slice of the list
    const int n_own = sh.slice_n[wv];
    for (int i = lane; i < n_own; i += 64) {
      const uint32_t rk = sh.list[wv][i];
      mine += rk >= thr ? weight_of(rk) : 0u;
    }
  } else {
    fence_row(rank);
#pragma unroll
    for (int c = 0; c < C; ++c) mine += kept(c);
  }
  const uint64_t wave_total = lane_u64(wave_scan_u64(mine), 63);
  if (lane == 0) sh.wave_part[wv] = wave_total;
  if (threadIdx.x == 0) sh.token = -1;
  __syncthreads();
  uint64_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kSampleWaves; ++i) {
    before += i < wv ? sh.wave_part[i] : 0;
    total += sh.wave_part[i];
  }
  uint64_t target = (uint64_t)((double)u * (double)total);
  target = target < total ? target : total - 1;   // u < 1, whatever the double rounding
  if (wave_total > 0 && before <= target && target < before + wave_total) {
    // rows in batches of up to four, whose scans are independent
    constexpr int kBatch = R < 4 ? R : 4;
    uint64_t acc = before;   // mass of the rows before the current batch
    fence_row(rank);
#pragma unroll
    for (int r0 = 0; r0 < R; r0 += kBatch) {
      uint64_t rs[kBatch], incl[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        rs[b] = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) rs[b] += kept((r0 + b) * G + j);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) incl[b] = wave_scan_u64(rs[b]);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const uint64_t ex = acc + incl[b] - rs[b];
        if (rs[b] > 0 && ex <= target && target < ex + rs[b]) {
          uint64_t g = ex;
          int tok = -1;
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const uint32_t k = kept((r0 + b) * G + j);
            if (tok < 0 && g + k > target) tok = token_of((r0 + b) * G + j);
            g += k;
          }
          sh.token = tok;
        }
        acc += lane_u64(incl[b], 63);
      }
      if (acc > target) break;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.tokens[row] = sh.token;
}

template <typename T>
hipError_t launch_rows(const SampleArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_rows), block(kSampleThreads);
  const int per_thread = (a.vocab + kSampleThreads - 1) / kSampleThreads;
  if (per_thread <= 1)
    hipLaunchKernelGGL((sample_kernel<T, 1>), grid, block, 0, stream, a);
  else if (per_thread <= 2)
    hipLaunchKernelGGL((sample_kernel<T, 2>), grid, block, 0, stream, a);
  else if (per_thread <= 4)
    hipLaunchKernelGGL((sample_kernel<T, 4>), grid, block, 0, stream, a);
  else if (per_thread <= 8)
    hipLaunchKernelGGL((sample_kernel<T, 8>), grid, block, 0, stream, a);
  else if (per_thread <= 16)
    hipLaunchKernelGGL((sample_kernel<T, 16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((sample_kernel<T, 32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs& a, bool bf16, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  if (a.vocab < 1 || a.vocab > kMaxSampleVocab) return hipErrorInvalidValue;
  return bf16 ? launch_rows<bf16_t>(a, stream) : launch_rows<float>(a, stream);
}

}  // namespace pa
