// Paged-attention decode on the vector ALUs: kernel templates.
//
// Included by decode_valu_bf16.hip, decode_valu_f32.hip and decode_valu_fp8.hip,
// which instantiate the kernels for one cache element type each (they compile
// in parallel), and by decode.hip for the element traits of the split-K merge.
// T is the query and output type (fp32 or bf16), KV the cache element type:
// T itself, or an FP8 (E4M3) code whose value is code * scale, the per-tensor
// scales folded into the score scale (K) and the output (V).
//
// What is computed: for every query row, softmax(scale * q K^T) V over the
// tokens of its sequence, K and V being read through the sequence's block table
// from the pool [num_blocks, num_kv_heads, block_size, head_dim] ("vLLM 基本原理",
// section PagedAttention; intelliparadigm.com article, section 3.1).  Decode
// re-reads the whole cache for one new token and is bound by memory bandwidth
// (xdnf.cn article, section 六.5), so the kernel is built around streaming the
// K/V blocks once at full width and hiding all arithmetic under those loads.
//
// Work decomposition.  One workgroup (4 waves) per (item, kv head, partition),
// kv heads varying fastest in launch order,
// where an item is a sequence (decode) or one prefill query token (the generic
// per-token prefill path).  A partition is a run of consecutive blocks; the
// waves of a workgroup take its blocks round-robin.  All query heads that share
// the kv head (a GQA group) are handled by the same workgroup, so each K/V
// block is read from HBM exactly once per step.  A plain split-K decode takes
// the same units from a schedule instead (decode_valu_dealt_kernel): longest
// partitions first, dealt to the XCDs by how fast each drains them.
//
// Lane layout inside a wave for one 16-token block slab (16 x head_dim values,
// contiguous in memory): every lane issues 16-byte loads; LPR = head_dim*elem/16
// lanes cover one token row, so a wave-wide load covers 64/LPR rows and a slab
// takes 16*LPR/64 loads per lane.  A lane's row group keeps its own online
// softmax state (running max m, running sum l, output slice acc) for the tokens
// it sees; the only per-token cross-lane step is the LPR-lane sum of the q.k
// partial dot products, done with DPP inside a 16-lane row.  Row groups, waves
// and partitions are merged once at the end with the log-sum-exp rule.
//
// Streaming.  Each wave keeps two slabs in flight (the next block's K/V loads
// are issued before the current block is consumed), the loads carry the
// nontemporal hint, and full blocks take a path without row masks; only a
// sequence's last, partly filled block pays for them.
//
// Scores are kept in base 2: q is pre-multiplied by scale*log2(e), so softmax
// weights are exp2(s - m), taken with the raw v_exp_f32 inside the block loop
// (weights below 2^-126 flush to zero, which a softmax ignores).
#pragma once

#include <math.h>

#include <type_traits>

#include "decode_groups.h"
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kWavesPerGroup = 4;

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<float> {
  static constexpr int kPerLoad = 4;
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
template <>
struct ElemTraits<bf16_t> {
  static constexpr int kPerLoad = 8;
  __device__ static float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
  __device__ static bf16_t from_f32(float x) { return f32_to_bf16(x); }
};
template <>
struct ElemTraits<fp8_t> {   // cache codes only: never a query or output type
  static constexpr int kPerLoad = 16;
};

// Widen the E elements held in one 16-byte register quad to fp32.
template <typename T>
__device__ __forceinline__ void widen(const u32x4& r, float* out);
template <>
__device__ __forceinline__ void widen<float>(const u32x4& r, float* out) {
#pragma unroll
  for (int x = 0; x < 4; ++x) out[x] = __uint_as_float(r[x]);
}
template <>
__device__ __forceinline__ void widen<bf16_t>(const u32x4& r, float* out) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    out[2 * x] = bf16_lo(r[x]);
    out[2 * x + 1] = bf16_hi(r[x]);
  }
}
template <>
__device__ __forceinline__ void widen<fp8_t>(const u32x4& r, float* out) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const uint32_t w = r[x];
    fp8x4_to_f32(w, out + 4 * x);
  }
}

// Partial q.k over this lane's E elements.  bf16 uses the packed bf16 dot
// instruction on the raw bits (q kept unscaled in bf16, products exact in fp32),
// fp32 uses fused multiply-adds on pre-scaled q.  FP8 keys are widened first,
// exactly (to bf16 pairs for a bf16 query, to fp32 for an fp32 query).
template <typename T, typename KV>
struct QFrag;
template <>
struct QFrag<float, float> {
  float q[4];
  __device__ void load(const float* p, float scale_log2) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int x = 0; x < 4; ++x) q[x] = __uint_as_float(r[x]) * scale_log2;
  }
  __device__ void zero() {
#pragma unroll
    for (int x = 0; x < 4; ++x) q[x] = 0.f;
  }
  __device__ float dot(const u32x4& k) const {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) s = fmaf(q[x], __uint_as_float(k[x]), s);
    return s;
  }
  __device__ static float post(float s, float) { return s; }
};
template <>
struct QFrag<bf16_t, bf16_t> {
  u32x4 q;
  __device__ void load(const bf16_t* p, float) { q = *reinterpret_cast<const u32x4*>(p); }
  __device__ void zero() { q = u32x4{0u, 0u, 0u, 0u}; }
  __device__ float dot(const u32x4& k) const {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t qw = q[x];
      const uint32_t kw = k[x];
      s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw), as_bf16x2(kw), s, false);
    }
    return s;
  }
  __device__ static float post(float s, float scale_log2) { return s * scale_log2; }
};
template <>
struct QFrag<bf16_t, fp8_t> {
  u32x4 q[2];   // 16 bf16 query elements, unscaled
  __device__ void load(const bf16_t* p, float) {
    q[0] = *reinterpret_cast<const u32x4*>(p);
    q[1] = *reinterpret_cast<const u32x4*>(p + 8);
  }
  __device__ void zero() { q[0] = q[1] = u32x4{0u, 0u, 0u, 0u}; }
  __device__ float dot(const u32x4& k) const {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t kw = k[x];
      const u32x2 kb = fp8x4_to_bf16x4(kw);
      const uint32_t q0 = q[x / 2][2 * (x % 2)];
      const uint32_t q1 = q[x / 2][2 * (x % 2) + 1];
      const uint32_t k0 = kb.x;
      const uint32_t k1 = kb.y;
      s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q0), as_bf16x2(k0), s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q1), as_bf16x2(k1), s, false);
    }
    return s;
  }
  __device__ static float post(float s, float scale_log2) { return s * scale_log2; }
};
template <>
struct QFrag<float, fp8_t> {
  float q[16];  // 16 fp32 query elements, pre-scaled
  __device__ void load(const float* p, float scale_log2) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const u32x4 r = *reinterpret_cast<const u32x4*>(p + 4 * x);
#pragma unroll
      for (int y = 0; y < 4; ++y) q[4 * x + y] = __uint_as_float(r[y]) * scale_log2;
    }
  }
  __device__ void zero() {
#pragma unroll
    for (int x = 0; x < 16; ++x) q[x] = 0.f;
  }
  __device__ float dot(const u32x4& k) const {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      float f[4];
      const uint32_t kw = k[x];
      fp8x4_to_f32(kw, f);
#pragma unroll
      for (int y = 0; y < 4; ++y) s = fmaf(q[4 * x + y], f[y], s);
    }
    return s;
  }
  __device__ static float post(float s, float) { return s; }
};

// One (block, kv head) slab of K and of V as this lane holds it: NLD
// 16-byte pieces each, rows RPL apart.
template <int NLD>
struct Slab {
  u32x4 k[NLD];
  u32x4 v[NLD];
};

// Slab loads go through a buffer resource per (block, kv head) slab: the base
// is the slab's address (scalar registers), lanes add 32-bit byte offsets, and
// the range check of the buffer unit turns a resource of size 0 into zero data
// with no memory access -- used for a lookahead past the last block and for
// block ids outside the pool.  A block that only this sequence reads is
// streamed with the nontemporal hint (measured ~10% faster than default
// caching on private KV); a block the caller marks as shared with other
// sequences of the call is read with the default policy, so sharers running
// at the same time hit in L2 (the shared-prefix decode runs ~1.5x faster).
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer, no format conversion
constexpr int kStreamPolicy = 2;           // cache-policy bits: nontemporal
constexpr int kSharedPolicy = 0;           // cache-policy bits: default

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
}

template <int POLICY>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t rsrc, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, byte_off, 0, POLICY);
}

template <typename KV, int D, int POLICY>
__device__ __forceinline__ void load_slab(Slab<kBlock * D / (kWave * ElemTraits<KV>::kPerLoad)>& s,
                                          __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                          int lane_byte_off) {
  constexpr int RPL = kWave / (D / ElemTraits<KV>::kPerLoad);
  constexpr int NLD = kBlock / RPL;
  constexpr int STEP = RPL * D * (int)sizeof(KV);
#pragma unroll
  for (int i = 0; i < NLD; ++i) s.k[i] = load16<POLICY>(kr, lane_byte_off + i * STEP);
#pragma unroll
  for (int i = 0; i < NLD; ++i) s.v[i] = load16<POLICY>(vr, lane_byte_off + i * STEP);
}

// Fold one slab into this lane's online-softmax state (running max m, running
// sum l, output slice acc per query head of the group).  MASKED: rows at or
// past nvalid are skipped -- their scores never enter the max, their weights
// are 0 and their V values are replaced by 0 before use, since they may hold
// anything (NaN included) and 0 * NaN is NaN.
template <typename T, typename KV, int D, int GP, bool MASKED>
__device__ __forceinline__ void consume_slab(
    const Slab<kBlock * D / (kWave * ElemTraits<KV>::kPerLoad)>& sl, const QFrag<T, KV> (&q)[GP],
    float scale_log2, int r, int nvalid, float (&m)[GP], float (&l)[GP],
    float (&acc)[GP][ElemTraits<KV>::kPerLoad]) {
  constexpr int E = ElemTraits<KV>::kPerLoad;
  constexpr int LPR = D / E;
  constexpr int RPL = kWave / LPR;
  constexpr int NLD = kBlock / RPL;

  // scores of this lane's rows, summed over the LPR lanes of each row
  float s[GP][NLD];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      s[g][i] = QFrag<T, KV>::post(group_sum<LPR>(q[g].dot(sl.k[i])), scale_log2);

  bool valid[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) valid[i] = !MASKED || i * RPL + r < nvalid;

  float p[GP][NLD];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      if (valid[i]) bm = fmaxf(bm, s[g][i]);
    const float mn = fmaxf(m[g], bm);
    // with masking, mn stays -inf while this row group has seen no token
    const float alpha = (MASKED && mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m[g] - mn);
    float lsum = l[g] * alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      p[g][i] = valid[i] ? __builtin_amdgcn_exp2f(s[g][i] - mn) : 0.f;
      lsum += p[g][i];
    }
    l[g] = lsum;
    m[g] = mn;
  }
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    u32x4 vr = sl.v[i];
    if (MASKED) vr = valid[i] ? vr : u32x4{0u, 0u, 0u, 0u};
    float v[E];
    widen<KV>(vr, v);
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p[g][i], v[e], acc[g][e]);
  }
}

// Locate the sequence an item belongs to and how many of its tokens it sees.
// Returns false if the item has no query row (past the last prefill token).
struct ItemInfo {
  int seq;
  int ctx;      // tokens visible to this item
  bool bad;     // contract violated: the item's outputs become NaN
};

__device__ __forceinline__ bool locate_item(const DecodeArgs& a, int item, ItemInfo& it) {
  if (a.query_start_loc == nullptr) {
    it.seq = item;
    it.ctx = a.context_lens[item];
    it.bad = it.ctx < 0 || it.ctx > a.max_blocks_per_seq * kBlock ||
             (a.partition_blocks > 0 && it.ctx > a.max_context_len);
    return true;
  }
  const int32_t* qsl = a.query_start_loc;
  if (item >= qsl[a.num_seqs] || item < qsl[0]) return false;
  int lo = 0, hi = a.num_seqs;  // invariant: qsl[lo] <= item < qsl[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qsl[mid] <= item) lo = mid; else hi = mid;
  }
  const int chunk = qsl[lo + 1] - qsl[lo];
  const int len = a.context_lens[lo];
  it.seq = lo;
  it.ctx = len - chunk + (item - qsl[lo]) + 1;
  // a non-monotone query_start_loc can leave item outside its chunk
  it.bad = item >= qsl[lo + 1] || chunk > len || chunk > a.max_query_len ||
           len > a.max_blocks_per_seq * kBlock || it.ctx < 1 || it.ctx > len;
  return true;
}

// LDS of one workgroup: each wave's merged state, for the merge of the waves.
template <int GP, int D>
struct ValuShared {
  float acc[kWavesPerGroup][GP][D];
  float m[kWavesPerGroup][GP];
  float l[kWavesPerGroup][GP];
  int bad[kWavesPerGroup];
  uint32_t mismatch[kWavesPerGroup];
};

// One work unit: kv head kvh of item `item`, partition `part` (the whole
// context without split-K).  Every thread of the workgroup calls it with the
// same unit; it returns early, all threads together, for units without work.
//
// HINT: the caller passed shared_prefix_blocks, so batches of shared blocks
// take the caching load path; without it only the streaming path is compiled.
// GROUPED: the grouped pass.  Workgroup (s, kv head, partition) works only if
// s opens a window of its group (s - leader a multiple of group_members) and
// the partition lies in the grouped prefix of some member of the window; the
// blocks come from the leader's table, query slot g is query head
// kvh*G + g % G of member s + g / G, and a member whose table names other
// blocks there gets NaN (it broke the grouping contract).
template <typename T, typename KV, int D, int GP, bool HINT, bool GROUPED>
__device__ __forceinline__ void decode_valu_unit(const DecodeArgs& a, const int item,
                                                 const int kvh, const int part,
                                                 ValuShared<GP, D>& sh) {
  constexpr int E = ElemTraits<KV>::kPerLoad;  // cache elements per 16-byte load
  constexpr int LPR = D / E;                   // lanes per token row
  constexpr int RPL = kWave / LPR;             // token rows per wave-wide load
  constexpr int NLD = kBlock / RPL;            // loads per block slab per lane
  constexpr int NW = kWavesPerGroup;
  static_assert(LPR >= 2 && LPR <= 32 && NLD >= 1, "layout");
  static_assert(!GROUPED || (GP <= 32 && !HINT), "grouped pass");

  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_uniform(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int G = a.group;
  const int hq = a.num_heads;
  T* out = static_cast<T*>(a.out);

  // This workgroup folds blocks [jb, je) of `table` (tokens below tok_end),
  // the first nshared of the sequence's table read with caching.
  int jb, je, tok_end, nshared;
  const int32_t* table;
  uint32_t active = 0;   // grouped: bit m = member item + m takes part
  int nparts = 1;        // regular: partitions of the item's sequence
  int seq = item;        // regular: the item's sequence
  if constexpr (GROUPED) {
    const int M = a.group_members;
    const int lead = a.prefix_group[item];
    if (lead < 0 || lead > item || (item - lead) % M != 0) return;
    for (int m = 0; m < M && item + m < a.num_seqs; ++m)
      if (a.prefix_group[item + m] == lead && part < grouped_parts(a, item + m))
        active |= 1u << m;
    if (active == 0) return;
    jb = part * a.partition_blocks;
    je = jb + a.partition_blocks;
    tok_end = je * kBlock;   // grouped partitions are whole blocks of every member
    nshared = 0;             // read once here: streamed
    table = a.block_tables + (int64_t)lead * a.max_blocks_per_seq;
  } else {
    ItemInfo it;
    if (!locate_item(a, item, it)) return;
    seq = it.seq;
    const int nblk = it.bad ? 0 : (it.ctx + kBlock - 1) / kBlock;
    const bool split = a.partition_blocks > 0;
    nparts = split ? (nblk + a.partition_blocks - 1) / a.partition_blocks : 1;
    if (part >= (nparts > 0 ? nparts : 1)) return;
    if (part < grouped_parts(a, it.seq)) return;   // the grouped pass wrote it
    jb = split ? part * a.partition_blocks : 0;
    je = split ? min(nblk, jb + a.partition_blocks) : nblk;
    tok_end = min(it.ctx, je * kBlock);

    // Degenerate items (only partition 0 gets here): no context gives zeros, a
    // violated contract gives NaN.
    if (it.bad || it.ctx == 0) {
      const float fill = it.bad ? __builtin_nanf("") : 0.f;
      if (split && it.bad && it.ctx > 0 && it.ctx <= a.max_context_len) {
        // the merge step will read this item's partitions: poison all of them
        const int ptok = a.partition_blocks * kBlock;
        const int np_bad = (it.ctx + ptok - 1) / ptok;
        if (np_bad > 1) {
          for (int i = threadIdx.x; i < np_bad * G * D; i += blockDim.x) {
            const int p = i / (G * D);
            const int g = (i / D) % G;
            const int64_t row = ((int64_t)it.seq * hq + kvh * G + g) * a.max_partitions + p;
            a.part_o[row * D + i % D] = fill;
            if (i % D == 0) a.part_lse[row] = fill;
          }
          return;
        }
      }
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        out[((int64_t)item * hq + kvh * G) * D + i] = ElemTraits<T>::from_f32(fill);
      return;
    }
    nshared = HINT ? a.shared_prefix_blocks[it.seq] : 0;
    table = a.block_tables + (int64_t)it.seq * a.max_blocks_per_seq;
  }

  // Query fragments of the slots: this lane's E elements of each.
  QFrag<T, KV> q[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    int64_t row = -1;
    if constexpr (GROUPED) {
      const int m = g / G;
      if ((active >> m) & 1u) row = (int64_t)(item + m) * hq + kvh * G + (g - m * G);
    } else {
      if (g < G) row = (int64_t)item * hq + kvh * G + g;
    }
    if (row >= 0)
      q[g].load(static_cast<const T*>(a.query) + row * D + c * E, a.scale_log2);
    else
      q[g].zero();
  }

  float m[GP], l[GP], acc[GP][E];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const KV* kpool = static_cast<const KV*>(a.k_cache);
  const KV* vpool = static_cast<const KV*>(a.v_cache);
  const int64_t head_slab = (int64_t)kBlock * D;
  const int lane_off = r * D + c * E;     // elements from the slab start
  bool bad_block = false;
  uint32_t mismatch = 0;                  // grouped: bit m = member m names other blocks

  // Blocks of this wave: jb + w, jb + w + NW, ...  Their ids are fetched up to
  // 64 at a time into one register (lane t holds the t-th) and broadcast per
  // step.  Two slabs are in flight: the next block's loads are issued before
  // the current block is consumed, unconditionally (straight-line code, so
  // each consume waits only for its own slab); past the last block of a batch
  // the resource is empty and the load moves no data.  A block id outside the
  // pool reads as zeros and poisons the result.  Batches never mix shared and
  // private blocks, so each batch runs with one cache policy.
  const int nb_w = (je - jb - w + NW - 1) / NW;
  const int slab_bytes = kBlock * D * (int)sizeof(KV);
  const int lane_byte_off = lane_off * (int)sizeof(KV);
  const int shared_ahead = nshared - jb - w;   // this wave's block idx is shared iff idx < idx_shared
  const int idx_shared = shared_ahead > 0 ? min(nb_w, (shared_ahead + NW - 1) / NW) : 0;
  for (int base = 0; base < nb_w;) {
    const bool shared_batch = base < idx_shared;
    const int cnt = min(kWave, (shared_batch ? idx_shared : nb_w) - base);
    const int jl = jb + w + NW * (base + lane);   // this lane's table entry
    const int myb = lane < cnt ? table[jl] : 0;
    if constexpr (GROUPED) {
#pragma unroll
      for (int mm = 0; mm < GP; ++mm)
        if ((active >> mm) & 1u) {
          const int32_t* tm = a.block_tables + (int64_t)(item + mm) * a.max_blocks_per_seq;
          if (lane < cnt && tm[jl] != myb) mismatch |= 1u << mm;
        }
    }
    const auto run_batch = [&](auto policy) {
      constexpr int P = decltype(policy)::value;
      const auto load_step = [&](Slab<NLD>& sl, int t) {
        const int bid = __builtin_amdgcn_readlane(myb, min(t, cnt - 1));
        const bool in_pool = bid >= 0 && (int64_t)bid < a.num_blocks;
        bad_block |= t < cnt && !in_pool;
        const bool live = t < cnt && in_pool;
        const int64_t off = live ? ((int64_t)bid * a.num_kv_heads + kvh) * head_slab : 0;
        const int bytes = live ? slab_bytes : 0;
        load_slab<KV, D, P>(sl, slab_rsrc(kpool + off, bytes), slab_rsrc(vpool + off, bytes),
                            lane_byte_off);
      };
      const auto consume = [&](const Slab<NLD>& sl, int t) {
        const int j = jb + w + NW * (base + t);
        const int nvalid = min(kBlock, tok_end - j * kBlock);
        if (nvalid == kBlock)
          consume_slab<T, KV, D, GP, false>(sl, q, a.scale_log2, r, nvalid, m, l, acc);
        else
          consume_slab<T, KV, D, GP, true>(sl, q, a.scale_log2, r, nvalid, m, l, acc);
      };
      Slab<NLD> sa, sb;
      load_step(sa, 0);
      for (int t = 0; t < cnt; t += 2) {
        load_step(sb, t + 1);
        consume(sa, t);
        if (t + 1 >= cnt) break;
        load_step(sa, t + 2);
        consume(sb, t + 1);
      }
    };
    if constexpr (HINT) {
      if (shared_batch)
        run_batch(std::integral_constant<int, kSharedPolicy>());
      else
        run_batch(std::integral_constant<int, kStreamPolicy>());
    } else {
      run_batch(std::integral_constant<int, kStreamPolicy>());
    }
    base += cnt;
  }

  // Merge the row groups of this wave (lanes that differ in index bits >= LPR).
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const float mw = xor_max_above<LPR>(m[g]);
    const float f = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - mw);
    l[g] = xor_sum_above<LPR>(l[g] * f);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = xor_sum_above<LPR>(acc[g][e] * f);
    m[g] = mw;
  }
  if constexpr (GROUPED) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) mismatch |= (uint32_t)__shfl_xor((int)mismatch, o, 64);
  }
  __syncthreads();
  if (lane == 0) {
    sh.bad[w] = __builtin_amdgcn_readfirstlane((int)bad_block);
    sh.mismatch[w] = mismatch;
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) sh.acc[w][g][c * E + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      sh.m[w][g] = m[g];
      sh.l[w][g] = l[g];
    }
  }
  __syncthreads();

  // Merge the waves and write this workgroup's results.
  bool poisoned = false;
  uint32_t mism = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    poisoned |= sh.bad[x] != 0;
    mism |= sh.mismatch[x];
  }
  const int nslots = GROUPED ? a.group_members * G : G;
  for (int i = threadIdx.x; i < nslots * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i - g * D;
    int oseq = seq, orow = item, h = kvh * G + g, np = nparts;
    bool bad = poisoned;
    if constexpr (GROUPED) {
      const int mm = g / G;
      if (!((active >> mm) & 1u)) continue;
      oseq = orow = item + mm;
      h = kvh * G + (g - mm * G);
      bad |= ((mism >> mm) & 1u) != 0;
      const int nblk = (a.context_lens[oseq] + kBlock - 1) / kBlock;
      np = (nblk + a.partition_blocks - 1) / a.partition_blocks;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < NW; ++x) mx = fmaxf(mx, sh.m[x][g]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const float f = (sh.m[x][g] == -INFINITY) ? 0.f : exp2f(sh.m[x][g] - mx);
      lsum = fmaf(sh.l[x][g], f, lsum);
      o = fmaf(sh.acc[x][g][d], f, o);
    }
    o = bad ? __builtin_nanf("") : o / lsum;
    if constexpr (std::is_same<KV, fp8_t>::value) o *= a.v_scale;
    if (np <= 1) {
      out[((int64_t)orow * hq + h) * D + d] = ElemTraits<T>::from_f32(o);
    } else {
      const int64_t row = ((int64_t)oseq * hq + h) * a.max_partitions + part;
      a.part_o[row * D + d] = o;
      if (d == 0) a.part_lse[row] = bad ? __builtin_nanf("") : (mx + log2f(lsum)) * kLn2;
    }
  }
}

// One workgroup per unit.  blockIdx.x = item * num_kv_heads + kv head:
// workgroups launched together read the adjacent head slabs of the same
// physical blocks, which keeps the HBM accesses of concurrently running waves
// close together.  The regular pass of a grouped call takes the partitions
// last first: its leading partitions are mostly the grouped ones it skips, and
// dispatched last their empty workgroups fill the launch's tail instead of
// holding slots the live ones need.  Otherwise the first (longest) partitions
// go first.
template <typename T, typename KV, int D, int GP, bool HINT, bool GROUPED>
__global__ __launch_bounds__(64 * kWavesPerGroup) void decode_valu_kernel(DecodeArgs a) {
  __shared__ ValuShared<GP, D> sh;
  const int item = blockIdx.x / a.num_kv_heads;
  const int kvh = blockIdx.x - item * a.num_kv_heads;
  const int part = (!GROUPED && a.prefix_group != nullptr) ? gridDim.y - 1 - blockIdx.y
                                                           : blockIdx.y;
  decode_valu_unit<T, KV, D, GP, HINT, GROUPED>(a, item, kvh, part, sh);
}

// Split-K decode over a dealt schedule.  The units are the (sequence,
// partition) pairs that decode_schedule_kernel, launched just before, sorted
// longest first, each followed by its kv heads; workgroup b takes unit
// dealt_unit(b).  So every XCD starts on long units and ends on short ones,
// and the even-numbered XCDs, which drain blocks faster, take more of them
// (decode_schedule_kernel's notes give the measurements); within an XCD the
// hardware hands the next workgroup to the first free slot.
template <typename T, typename KV, int D, int GP>
__global__ __launch_bounds__(64 * kWavesPerGroup) void decode_valu_dealt_kernel(DecodeArgs a) {
  __shared__ ValuShared<GP, D> sh;
  const int nkv = a.num_kv_heads;
  const int t = dealt_unit(blockIdx.x);
  if (t >= a.sched[kSchedPairs] * nkv) return;
  const int* const pairs = a.sched + kSchedHeader;
  const int u = t / nkv;
  const int pair = pairs[u];
  const int item = pair / a.max_partitions;
  decode_valu_unit<T, KV, D, GP, false, false>(a, item, t - u * nkv,
                                               pair - item * a.max_partitions, sh);
}

// Query heads per kv head the vector-ALU kernel takes for an FP8 cache: its
// widened fp32 accumulators (16 per head and lane) leave no room for more.
constexpr int kFp8ValuMaxGroup = 4;

template <typename T, typename KV, int D, bool HINT>
inline void launch_decode_group(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * kWavesPerGroup);
  const int G = a.group;
  if (G <= 1)
    hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 1, HINT, false>), grid, block, 0, stream, a);
  else if (G <= 2)
    hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 2, HINT, false>), grid, block, 0, stream, a);
  else if (G <= 4)
    hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 4, HINT, false>), grid, block, 0, stream, a);
  else if constexpr (!std::is_same<KV, fp8_t>::value) {
    if (G <= 8)
      hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 8, HINT, false>), grid, block, 0, stream,
                         a);
    else
      hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 16, HINT, false>), grid, block, 0, stream,
                         a);
  }
}

// The grouped pass, with the fewest slots that hold a window's queries.
template <typename T, typename KV, int D>
inline void launch_decode_grouped(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * kWavesPerGroup);
  const int slots = a.group_members * a.group;
  if (slots <= 2)
    hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 2, false, true>), grid, block, 0, stream, a);
  else if (slots <= 3)
    hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 3, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, 4, false, true>), grid, block, 0, stream, a);
}

// The dealt split-K decode: decode_schedule_kernel, then one workgroup per
// slot of the deal.
template <typename T, typename KV, int D>
inline hipError_t launch_decode_dealt(const DecodeArgs& a, hipStream_t stream) {
  const hipError_t e = launch_decode_schedule(a, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)deal_blocks((int64_t)a.num_items * a.max_partitions * a.num_kv_heads));
  const dim3 block(64 * kWavesPerGroup);
  if (a.group <= 1)
    hipLaunchKernelGGL((decode_valu_dealt_kernel<T, KV, D, 1>), grid, block, 0, stream, a);
  else if (a.group <= 2)
    hipLaunchKernelGGL((decode_valu_dealt_kernel<T, KV, D, 2>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu_dealt_kernel<T, KV, D, 4>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <typename T, typename KV, int D>
inline hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  if (std::is_same<KV, fp8_t>::value && a.group > kFp8ValuMaxGroup) return hipErrorInvalidValue;
  dim3 grid((unsigned)((int64_t)a.num_items * a.num_kv_heads),
            a.partition_blocks > 0 ? a.max_partitions : 1);
  DecodeArgs b = a;   // both passes see the same window size
  b.group_members = group_window(a, kGroupedMaxSlots);
  if (b.group_members == 0) b.prefix_group = nullptr;
  if (b.prefix_group != nullptr) {
    if (b.partition_blocks <= 0 || b.shared_prefix_blocks == nullptr ||
        b.query_start_loc != nullptr)
      return hipErrorInvalidValue;
    launch_decode_grouped<T, KV, D>(b, grid, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // A plain split-K decode with up to four query heads per kv head runs over
  // the dealt schedule (while its units stay well inside an int).
  if (b.prefix_group == nullptr && b.shared_prefix_blocks == nullptr &&
      b.query_start_loc == nullptr && b.partition_blocks > 0 && b.sched != nullptr &&
      b.group <= 4 &&
      (int64_t)b.num_items * b.max_partitions * b.num_kv_heads < (int64_t(1) << 30))
    return launch_decode_dealt<T, KV, D>(b, stream);
  if (b.shared_prefix_blocks != nullptr)
    launch_decode_group<T, KV, D, true>(b, grid, stream);
  else
    launch_decode_group<T, KV, D, false>(b, grid, stream);
  return hipGetLastError();
}

}  // namespace pa
