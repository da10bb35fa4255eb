// Paged-attention decode for grouped-query heads on bf16 matrix cores (MFMA).
//
// Same computation as the vector-ALU decode: for each query head h of a
// sequence, softmax(scale * q_h K^T) V over the sequence's cached tokens, K and
// V read through the block table from the pool [num_blocks, num_kv_heads,
// block_size, head_dim] ("vLLM 基本原理", section PagedAttention;
// intelliparadigm.com article, section 3.1).  When G = num_heads / num_kv_heads
// query heads share one kv head, every K/V row meets G queries, so q.K^T and
// p.V become small dense products: S^T = K Q^T (16 tokens x G heads, reduced
// over head_dim) and O^T = V^T P^T (head_dim x G heads, reduced over tokens).
// Decode stays bound by HBM (xdnf.cn article, section 六.5): the matrix cores
// only take the arithmetic off the vector ALUs so that the loads are never
// starved.
//
// Work decomposition.  One wave per (sequence, kv head, partition), and one
// wave per workgroup, kv heads fastest in launch order: the waves of one
// (sequence, partition) walk the same block ids and read neighbouring 4 KiB
// head slabs.  Waves never exchange data: each owns its heads' whole softmax
// state, and partitions meet in the split-K merge.  Single-wave workgroups
// measured faster than workgroups of 2, 4 or 8 kv heads (476 / 495 / 503 /
// 534 us on the Llama-3-8B-shaped batch, 254 / 274 / 284 / 295 us over an FP8
// cache).  A split-K call with no grouped pass (and at most 64 sequences)
// runs the same waves persistently instead: as many as stay resident walk the
// ids and hold their partials in LDS until their walk is done (see the
// kernel), 487 -> 449 us on that batch.
//
// Operand layouts (v_mfma_f32_16x16x32_bf16 for scores, v_mfma_f32_16x16x16_bf16
// for p.V).  In both, lane l = 16 g + r supplies row/column r and reduction
// slots [8g, 8g+8) resp. [4g, 4g+4); a 16x16 result leaves rows 4g .. 4g+3 of
// column r in lane l.
//  - K is the A operand of the score product with token r in row r.  The
//    reduction order over head_dim is free as long as Q uses the same one, so
//    lane (r, g) takes 16-byte chunk 4ks + g of token r at k-step ks.  Loading
//    that pattern straight from memory (16 rows touched per instruction) runs
//    well below the HBM rate, so K is loaded exactly like V (16 lanes per
//    contiguous 256-byte row) and turned around through a small per-wave LDS
//    tile: 4 16-byte writes and 4 16-byte reads per lane and block, rows
//    padded to 272 bytes so neither side has bank conflicts.
//  - Q^T is the B operand: lane (r, g) holds chunk 4ks + g of query head r
//    (zero for r >= G).
//  - The score result leaves tokens 4g .. 4g+3 of head r in lane (r, g): the
//    softmax state of head r lives in the 4 lanes r, r+16, r+32, r+48, and its
//    probabilities are already laid out as the B operand of p.V (P^T).
//  - V is the A operand of O^T = V^T P^T, where row r of d-tile t stands for
//    column 8r + t.  Lane (r, g) loads columns 8r .. 8r+7 of tokens 4g .. 4g+3
//    (one fully contiguous 256-byte row per 16 lanes and instruction) and
//    takes element t of each of the four loads as its operand for tile t, a
//    register-local repack.  Output tile t then holds columns 8(4g+i) + t in
//    lane (r, g), so every lane ends with 4 runs of 8 consecutive columns.
//
// Scores are kept in base 2 (scale * log2(e)); probabilities are rounded to
// bf16 for the p.V product and the running sum adds the rounded values, so
// numerator and denominator use the same weights.
//
// FP8 (E4M3) caches: each lane loads the same token rows and columns as for
// bf16, 8 bytes instead of 16, and widens the codes to bf16 in registers when
// it consumes the slab (exact: an E4M3 value has at most 4 significant bits);
// from there the products are the bf16 ones.  The per-tensor K scale is folded
// into the score scale, the V scale into the final normalisation.
#include <math.h>

#include <type_traits>

#include "decode_groups.h"
#include <atomic>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kD = 128;          // head_dim handled here
constexpr int kHeadsPerWG = 1;   // kv heads (= waves) per workgroup
constexpr float kRescaleSlack = 8.f;   // base-2 headroom of the lazy softmax rescale

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_qk(const u32x4& k, const u32x4& q, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                 __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_pv(const u32x2& v, const u32x2& p, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, v),
                                                   __builtin_bit_cast(i16x4, p), c, 0, 0, 0);
}

// Loads go through a buffer resource per slab (base = the slab's address,
// lanes add byte offsets); a resource of size 0 yields zeros with no memory
// access, used for a lookahead past the last block and for block ids outside
// the pool.  Blocks only this sequence reads are streamed (nontemporal hint);
// blocks the caller marks as shared with other sequences use the default
// policy so that concurrent sharers hit in L2.
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
template <int POLICY>
__device__ __forceinline__ u32x2 load8(__amdgpu_buffer_rsrc_t rsrc, int byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, byte_off, 0, POLICY));
}

// K and V of one (block, kv head) slab as this lane holds them: token 4g+i,
// columns 8r .. 8r+7 (16 lanes per contiguous row), as bf16 ...
struct MfmaSlab {
  u32x4 k[4];
  u32x4 v[4];
};
// ... and as loaded from an FP8 cache (8 codes per token row and lane).
struct MfmaSlabFp8 {
  u32x2 k[4];
  u32x2 v[4];
};

template <typename KV>
using SlabOf = typename std::conditional<std::is_same<KV, fp8_t>::value, MfmaSlabFp8, MfmaSlab>::type;

template <typename KV, int POLICY>
__device__ __forceinline__ void load_mfma_slab(SlabOf<KV>& s, __amdgpu_buffer_rsrc_t kr,
                                               __amdgpu_buffer_rsrc_t vr, int r, int g) {
  constexpr int EB = (int)sizeof(KV);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = EB * ((4 * g + i) * kD + 8 * r);
    if constexpr (EB == 1) s.k[i] = load8<POLICY>(kr, off);
    else s.k[i] = load16<POLICY>(kr, off);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = EB * ((4 * g + i) * kD + 8 * r);
    if constexpr (EB == 1) s.v[i] = load8<POLICY>(vr, off);
    else s.v[i] = load16<POLICY>(vr, off);
  }
}

// The slab as bf16: the loaded registers themselves, or the FP8 codes widened.
__device__ __forceinline__ MfmaSlab& as_bf16_slab(MfmaSlab& s) { return s; }
__device__ __forceinline__ MfmaSlab as_bf16_slab(const MfmaSlabFp8& s) {
  MfmaSlab b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t k0 = s.k[i].x, k1 = s.k[i].y, v0 = s.v[i].x, v1 = s.v[i].y;
    const u32x2 klo = fp8x4_to_bf16x4(k0), khi = fp8x4_to_bf16x4(k1);
    const u32x2 vlo = fp8x4_to_bf16x4(v0), vhi = fp8x4_to_bf16x4(v1);
    b.k[i] = u32x4{klo.x, klo.y, khi.x, khi.y};
    b.v[i] = u32x4{vlo.x, vlo.y, vhi.x, vhi.y};
  }
  return b;
}

// Per-wave LDS tile that turns K around: 16 token rows of 256 bytes, padded.
constexpr int kKRowBytes = kD * 2 + 16;
constexpr int kKTileBytes = kBlock * kKRowBytes;

// Orders this wave's LDS accesses around a turn-around (LDS operations of one
// wave complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The low (t even) or high (t odd) bf16 of word w of two registers, packed as
// (hi_src << 16) | lo_src.
template <int T>
__device__ __forceinline__ uint32_t pick_pair(const u32x4& lo_src, const u32x4& hi_src) {
  const uint32_t sel = (T & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t lo = lo_src[T / 2];
  const uint32_t hi = hi_src[T / 2];
  return __builtin_amdgcn_perm(hi, lo, sel);
}

struct HeadState {
  float m;        // reference max (base-2 scores) of head r, same in its 4 lanes
  float lsum;     // this lane's share of the running sum
  f32x4 o[8];     // O^T tiles: o[t][i] is column 8(4g+i) + t of head r
};

// Fold one slab into the state.  Tokens at or past nvalid (only in a
// sequence's last block) are skipped: score -inf, weight 0, and their V rows
// replaced by zero in place, since they may hold anything and 0 * NaN is NaN.
// The masking only edits the inputs inside a uniform branch, so the
// accumulators keep one register assignment.  Token 0 of a block is always
// valid, so the block max is finite and the first block sets the reference.
__device__ __forceinline__ void consume_mfma_slab(MfmaSlab& sl, const u32x4 (&qb)[4],
                                                  float scale_log2, int r, int g, int nvalid,
                                                  uint8_t* ktile, HeadState& st) {
  // K into A-operand layout: write row 4g+i / chunk r, read row r / chunk 4ks+g.
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4*>(ktile + (4 * g + i) * kKRowBytes + 16 * r) = sl.k[i];
  wave_lds_sync();
  u32x4 ka[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    ka[ks] = *reinterpret_cast<const u32x4*>(ktile + r * kKRowBytes + 16 * (4 * ks + g));

  f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) sc = mfma_qk(ka[ks], qb[ks], sc);

  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = sc[i] * scale_log2;
  if (nvalid < kBlock) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = 4 * g + i < nvalid;
      s[i] = ok ? s[i] : -INFINITY;
      sl.v[i] = ok ? sl.v[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Lazy rescaling: the reference max st.m only moves when a score exceeds it
  // by more than kRescaleSlack, so weights stay <= 2^kRescaleSlack and the
  // accumulators are rescaled only then -- in practice on the first block and
  // rarely after.  Each lane checks its own 4 scores and the wave votes; the
  // head's max over its 4 lanes is gathered only inside that rare branch.
  // The result does not depend on the reference: out = o / lsum and
  // lse = st.m + log2(lsum).
  const float lmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  if (__ballot(lmax > st.m + kRescaleSlack) != 0) {
    float bm = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = bm > st.m + kRescaleSlack ? bm : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.lsum *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
    st.m = mn;
  }
  // raw v_exp_f32: weights below 2^-126 flush to zero, which a softmax ignores
  const float mr = st.m;
  const uint32_t p01 = pack_bf16x2(__builtin_amdgcn_exp2f(s[0] - mr),
                                   __builtin_amdgcn_exp2f(s[1] - mr));
  const uint32_t p23 = pack_bf16x2(__builtin_amdgcn_exp2f(s[2] - mr),
                                   __builtin_amdgcn_exp2f(s[3] - mr));
  st.lsum += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));

  const u32x2 pb = u32x2{p01, p23};
#define PA_PV_TILE(T)                                                               \
  st.o[T] = mfma_pv(u32x2{pick_pair<T>(sl.v[0], sl.v[1]), pick_pair<T>(sl.v[2], sl.v[3])}, \
                    pb, st.o[T]);
  PA_PV_TILE(0) PA_PV_TILE(1) PA_PV_TILE(2) PA_PV_TILE(3)
  PA_PV_TILE(4) PA_PV_TILE(5) PA_PV_TILE(6) PA_PV_TILE(7)
#undef PA_PV_TILE
}

}  // namespace

// KV: the cache element type (bf16, or fp8 codes).  HINT: the caller passed
// shared_prefix_blocks, so batches of shared blocks take the caching load path;
// without it only the streaming path is compiled.
template <typename KV, bool HINT, bool GROUPED, bool PERSIST>
__global__ __launch_bounds__(64 * kHeadsPerWG) void decode_gqa_mfma_kernel(DecodeArgs a) {
  static_assert(!(PERSIST && GROUPED), "persistent waves walk the regular pass only");
  __shared__ __attribute__((aligned(16))) uint8_t sh_k[kHeadsPerWG][kKTileBytes];
  const int hgroups = (a.num_kv_heads + kHeadsPerWG - 1) / kHeadsPerWG;
  // PERSIST (the regular pass of a split-K call without a grouped pass, at
  // most 64 sequences): a grid of resident waves walks the (sequence,
  // partition, kv head group) ids that have work, numbered densely --
  // sequence by sequence, its partitions, its head groups -- and dealt to the
  // waves in turn, so that every wave gets the same count.  Lane l holds
  // sequence l's partition count and, after a scan, the partitions before it.
  int cum_excl = 0;
  int64_t total = 1;
  if constexpr (PERSIST) {
    const int l = threadIdx.x & (kWave - 1);
    int np_l = 0;
    if (l < a.num_items) {
      const int ctx = a.context_lens[l];
      const bool bad_l = ctx < 0 || ctx > a.max_blocks_per_seq * kBlock || ctx > a.max_context_len;
      const int nb = bad_l ? 0 : (ctx + kBlock - 1) / kBlock;
      np_l = max(1, (nb + a.partition_blocks - 1) / a.partition_blocks);
    }
    int c = np_l;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(c, o, kWave);
      if (l >= o) c += y;
    }
    cum_excl = c - np_l;
    total = (int64_t)__shfl(c, a.num_items - 1, kWave) * hgroups;
  }
  // A persistent wave keeps its ids' split-K partials in LDS (up to 4 ids) and
  // writes them, whole rows per instruction, when its slots are full or its
  // ids are done.  Written at the end of each id, the partials cost the K/V
  // stream about 10% (21 MB among 2.8 GB at the GQA batch's 512-token
  // partitions), far more than their bytes, however they were laid out;
  // staged, most of them reach HBM after the stream.  Slot s holds the rows of
  // query heads kvh * G + hr at part_o rows sh_meta[s] + hr * max_partitions.
  constexpr int kStageFloats = PERSIST ? 2048 : 1;   // 8 KB per wave
  __shared__ float sh_stage[kHeadsPerWG][kStageFloats];
  __shared__ float sh_slse[kHeadsPerWG][PERSIST ? 64 : 1];
  __shared__ int64_t sh_meta[kHeadsPerWG][PERSIST ? 16 : 1];
  const int slot_floats = a.group * kD;
  const int slots = PERSIST ? min(4, kStageFloats / slot_floats) : 0;   // 1..4 for groups 4..16
  int used = 0;   // wave-uniform
  const auto flush_all = [&]() {
    if constexpr (PERSIST) {
      const int fl = threadIdx.x & (kWave - 1);
      const int wv = wave_uniform(threadIdx.x >> 6);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int sl = 0; sl < used; ++sl) {
        const int64_t base = sh_meta[wv][sl];
        const float* src = &sh_stage[wv][sl * slot_floats];
        for (int idx = 4 * fl; idx < slot_floats; idx += 4 * kWave) {
          const int64_t row = base + (int64_t)(idx / kD) * a.max_partitions;
          *reinterpret_cast<f32x4*>(a.part_o + row * kD + idx % kD) =
              *reinterpret_cast<const f32x4*>(src + idx);
        }
        if (fl < a.group)
          a.part_lse[base + (int64_t)fl * a.max_partitions] = sh_slse[wv][sl * 16 + fl];
      }
      __builtin_amdgcn_wave_barrier();
      used = 0;
    }
  };
  for (int64_t v = PERSIST ? (int64_t)blockIdx.x : 0; v < total; v += PERSIST ? gridDim.x : 1) {
  int item, by, hg;
  if constexpr (PERSIST) {
    const int t = (int)(v / hgroups);
    hg = (int)(v - (int64_t)t * hgroups);
    const int sl = threadIdx.x & (kWave - 1);
    const uint64_t below = __ballot(sl < a.num_items && cum_excl <= t);
    item = 63 - __builtin_clzll(below);
    by = t - __shfl(cum_excl, item, kWave);
  } else {
    item = blockIdx.x / hgroups;
    hg = blockIdx.x - item * hgroups;
    by = blockIdx.y;
  }
  const int kvh = hg * kHeadsPerWG + wave_uniform(threadIdx.x >> 6);
  // the regular pass of a grouped call takes the partitions last first (its
  // leading ones are mostly grouped: their empty workgroups then fill the tail)
  const int part = (!GROUPED && !PERSIST && a.prefix_group != nullptr) ? gridDim.y - 1 - by : by;
  if (kvh >= a.num_kv_heads) continue;
  int tix = threadIdx.x;
  if constexpr (PERSIST) __asm__ volatile("" : "+v"(tix));   // recomputed per id, not held
  const int lane = tix & (kWave - 1);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int G = a.group;
  const int hq = a.num_heads;
  bf16_t* out = static_cast<bf16_t*>(a.out);

  // This wave folds blocks [jb, je) of `table` (tokens below tok_end).  Column
  // r of the products is query head kvh*G + r of sequence item (regular), or
  // query head kvh*G + r % G of member item + r / G of a sharing window
  // (grouped: the blocks come from the leader's table, and a member whose
  // table names other blocks there gets NaN).
  int jb, je, tok_end, nparts = 1, nshared = 0;
  const int32_t* table;
  uint32_t active = 0;
  if constexpr (GROUPED) {
    const int M = a.group_members;
    const int lead = a.prefix_group[item];
    if (lead < 0 || lead > item || (item - lead) % M != 0) continue;
    for (int m = 0; m < M && item + m < a.num_seqs; ++m)
      if (a.prefix_group[item + m] == lead && part < grouped_parts(a, item + m))
        active |= 1u << m;
    if (active == 0) continue;
    jb = part * a.partition_blocks;
    je = jb + a.partition_blocks;
    tok_end = je * kBlock;
    table = a.block_tables + (int64_t)lead * a.max_blocks_per_seq;
  } else {
    const int ctx = a.context_lens[item];
    const bool bad = ctx < 0 || ctx > a.max_blocks_per_seq * kBlock ||
                     (a.partition_blocks > 0 && ctx > a.max_context_len);
    const int nblk = bad ? 0 : (ctx + kBlock - 1) / kBlock;
    const bool split = a.partition_blocks > 0;
    nparts = split ? (nblk + a.partition_blocks - 1) / a.partition_blocks : 1;
    if (part >= (nparts > 0 ? nparts : 1)) continue;
    if (part < grouped_parts(a, item)) continue;   // the grouped pass wrote it

    // Degenerate sequences (only partition 0 gets here): no context gives zeros,
    // a violated contract gives NaN, in the partials too if the merge will read
    // them.
    if (bad || ctx == 0) {
      const float fill = bad ? __builtin_nanf("") : 0.f;
      if (split && bad && ctx > 0 && ctx <= a.max_context_len) {
        const int ptok = a.partition_blocks * kBlock;
        const int np_bad = (ctx + ptok - 1) / ptok;
        if (np_bad > 1) {
          for (int i = lane; i < np_bad * G * kD; i += kWave) {
            const int p = i / (G * kD);
            const int h = (i / kD) % G;
            const int64_t row = ((int64_t)item * hq + kvh * G + h) * a.max_partitions + p;
            a.part_o[row * kD + i % kD] = fill;
            if (i % kD == 0) a.part_lse[row] = fill;
          }
          continue;
        }
      }
      for (int i = lane; i < G * kD; i += kWave)
        out[((int64_t)item * hq + kvh * G) * kD + i] = f32_to_bf16(fill);
      continue;
    }
    jb = split ? part * a.partition_blocks : 0;
    je = split ? min(nblk, jb + a.partition_blocks) : nblk;
    tok_end = min(ctx, je * kBlock);
    nshared = HINT ? a.shared_prefix_blocks[item] : 0;
    table = a.block_tables + (int64_t)item * a.max_blocks_per_seq;
  }
  // this lane's column: sequence colseq, query head colh (colseq < 0: no head)
  int colseq = -1, colh = 0;
  if constexpr (GROUPED) {
    const int m = r / G;
    if (m < 32 && ((active >> m) & 1u)) {
      colseq = item + m;
      colh = kvh * G + (r - m * G);
    }
  } else {
    if (r < G) {
      colseq = item;
      colh = kvh * G + r;
    }
  }

  u32x4 qb[4];
  const bf16_t* qrow =
      static_cast<const bf16_t*>(a.query) + ((int64_t)max(colseq, 0) * hq + colh) * kD;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qb[ks] = colseq >= 0 ? *reinterpret_cast<const u32x4*>(qrow + (4 * ks + g) * 8)
                         : u32x4{0u, 0u, 0u, 0u};

  HeadState st;
  st.m = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const KV* kpool = static_cast<const KV*>(a.k_cache);
  const KV* vpool = static_cast<const KV*>(a.v_cache);
  constexpr int kSlabBytes = kBlock * kD * (int)sizeof(KV);
  const int64_t head_slab = (int64_t)kBlock * kD;
  uint8_t* ktile = sh_k[kvh % kHeadsPerWG];
  bool bad_block = false;
  uint32_t mismatch = 0;   // grouped: bit m = member m names other blocks

  // Blocks jb .. je-1, their ids fetched 64 at a time (lane t holds the t-th)
  // and broadcast per step.  Two slabs are in flight: the next block's loads
  // are issued before the current one is consumed, unconditionally
  // (straight-line code, so each consume waits only for its own slab); past
  // the last block the resource is empty and the load moves no data.  An id
  // outside the pool reads as zeros and poisons the result.
  // Batches never mix blocks the caller marks as shared with private ones, so
  // each batch runs with one cache policy.
  const int shared_end = max(jb, min(je, nshared));
  for (int base = jb; base < je;) {
    const bool shared_batch = base < shared_end;
    const int cnt = min(kWave, (shared_batch ? shared_end : je) - base);
    const int myb = lane < cnt ? table[base + lane] : 0;
    if constexpr (GROUPED) {
      for (int m = 0; m < a.group_members; ++m)
        if ((active >> m) & 1u) {
          const int32_t* tm = a.block_tables + (int64_t)(item + m) * a.max_blocks_per_seq;
          if (lane < cnt && tm[base + lane] != myb) mismatch |= 1u << m;
        }
    }
    const auto run_batch = [&](auto policy) {
      constexpr int P = decltype(policy)::value;
      const auto load_step = [&](SlabOf<KV>& sl, int t) {
        const int bid = __builtin_amdgcn_readlane(myb, min(t, cnt - 1));
        const bool in_pool = bid >= 0 && (int64_t)bid < a.num_blocks;
        bad_block |= t < cnt && !in_pool;
        const bool live = t < cnt && in_pool;
        const int64_t off = live ? ((int64_t)bid * a.num_kv_heads + kvh) * head_slab : 0;
        const int bytes = live ? kSlabBytes : 0;
        load_mfma_slab<KV, P>(sl, slab_rsrc(kpool + off, bytes), slab_rsrc(vpool + off, bytes), r,
                              g);
      };
      const auto consume = [&](SlabOf<KV>& sl, int t) {
        const int nvalid = min(kBlock, tok_end - (base + t) * kBlock);
        auto&& bs = as_bf16_slab(sl);
        consume_mfma_slab(bs, qb, a.scale_log2, r, g, nvalid, ktile, st);
      };
      SlabOf<KV> sa, sb;
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

  // Head r's full sum is spread over its 4 lanes.  bad_block is the same in
  // every lane (block ids are broadcast).
  float lsum = st.lsum;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  bool poisoned = __builtin_amdgcn_readfirstlane((int)bad_block) != 0;
  int np = nparts;
  if constexpr (GROUPED) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) mismatch |= (uint32_t)__shfl_xor((int)mismatch, o, 64);
    if (colseq >= 0) {
      poisoned |= ((mismatch >> (r / G)) & 1u) != 0;
      const int nb = (a.context_lens[colseq] + kBlock - 1) / kBlock;
      np = (nb + a.partition_blocks - 1) / a.partition_blocks;
    }
  }
  if constexpr (PERSIST) {
    if (np > 1 && used >= slots) flush_all();
  }
  if (colseq >= 0) {
  float inv = 1.f / lsum;
  if constexpr (std::is_same<KV, fp8_t>::value) inv = a.v_scale / lsum;
  const int h = colh;
  if (np <= 1) {
    bf16_t* dst = out + ((int64_t)colseq * hq + h) * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 w;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        w[x] = poisoned ? 0x7FC07FC0u
                        : pack_bf16x2(st.o[2 * x][i] * inv, st.o[2 * x + 1][i] * inv);
      *reinterpret_cast<u32x4*>(dst + 8 * (4 * g + i)) = w;
    }
  } else {
    const int64_t row = ((int64_t)colseq * hq + h) * a.max_partitions + part;
    float* dst = PERSIST ? &sh_stage[wave_uniform(threadIdx.x >> 6)][used * slot_floats + r * kD]
                         : a.part_o + row * kD;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 lo, hi;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        lo[x] = poisoned ? nan : st.o[x][i] * inv;
        hi[x] = poisoned ? nan : st.o[4 + x][i] * inv;
      }
      *reinterpret_cast<f32x4*>(dst + 8 * (4 * g + i)) = lo;
      *reinterpret_cast<f32x4*>(dst + 8 * (4 * g + i) + 4) = hi;
    }
    const float lse = poisoned ? nan : (st.m + log2f(lsum)) * kLn2;
    if (g == 0) {
      if constexpr (PERSIST) sh_slse[wave_uniform(threadIdx.x >> 6)][used * 16 + r] = lse;
      else a.part_lse[row] = lse;
    }
  }
  }
  if constexpr (PERSIST) {
    if (np > 1) {
      if ((threadIdx.x & (kWave - 1)) == 0)
        sh_meta[wave_uniform(threadIdx.x >> 6)][used] =
            ((int64_t)item * hq + kvh * G) * a.max_partitions + part;
      ++used;
    }
  }
  }
  flush_all();
}

// Query columns of the products: a grouped-pass wave stacks the query heads
// of up to 16 / G sharers.
constexpr int kMfmaColumns = 16;

template <typename KV>
hipError_t launch_gqa_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  const int hgroups = (a.num_kv_heads + kHeadsPerWG - 1) / kHeadsPerWG;
  dim3 grid((unsigned)((int64_t)a.num_items * hgroups),
            a.partition_blocks > 0 ? a.max_partitions : 1);
  const dim3 block(64 * kHeadsPerWG);
  DecodeArgs b = a;   // both passes see the same window size
  b.group_members = group_window(a, kMfmaColumns);
  if (b.group_members == 0) b.prefix_group = nullptr;
  if (b.prefix_group != nullptr) {
    if (b.partition_blocks <= 0 || b.shared_prefix_blocks == nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_gqa_mfma_kernel<KV, false, true, false>), grid, block, 0, stream, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // (bf16 caches: over FP8 codes the same walk measured slower, 257 -> 294 us
  // on the GQA batch, and the launch stays one wave per id)
  if constexpr (std::is_same<KV, bf16_t>::value) {
    if (b.prefix_group == nullptr && b.partition_blocks > 0 && b.num_items <= kWave &&
        b.group >= 4 && b.group <= 16) {
      // split-K without a grouped pass: as many waves as stay resident walk
      // the ids and keep their partials until their walk ends (the count comes
      // from the occupancy the compiled kernel allows, once per device)
      static std::atomic<int> resident_cache[2][64];
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
      const int hint = b.shared_prefix_blocks != nullptr ? 1 : 0;
      int resident = resident_cache[hint][dev].load(std::memory_order_relaxed);
      if (resident <= 0) {
        int per_cu = 0, cus = 0;
        const hipError_t e1 = hint ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                         &per_cu, decode_gqa_mfma_kernel<KV, true, false, true>,
                                         64 * kHeadsPerWG, 0)
                                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                         &per_cu, decode_gqa_mfma_kernel<KV, false, false, true>,
                                         64 * kHeadsPerWG, 0);
        const hipError_t e2 =
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        const bool known = e1 == hipSuccess && e2 == hipSuccess && per_cu > 0 && cus > 0;
        resident = known ? per_cu * cus : 2048;
        resident = resident / 8 * 8;
        if (resident < 8) resident = 8;
        resident_cache[hint][dev].store(resident, std::memory_order_relaxed);
      }
      const int64_t ids = (int64_t)grid.x * grid.y;
      const dim3 pgrid((unsigned)(ids < resident ? ids : resident));
      if (hint)
        hipLaunchKernelGGL((decode_gqa_mfma_kernel<KV, true, false, true>), pgrid, block, 0,
                           stream, b);
      else
        hipLaunchKernelGGL((decode_gqa_mfma_kernel<KV, false, false, true>), pgrid, block, 0,
                           stream, b);
      return hipGetLastError();
    }
  }
  if (b.shared_prefix_blocks != nullptr)
    hipLaunchKernelGGL((decode_gqa_mfma_kernel<KV, true, false, false>), grid, block, 0, stream, b);
  else
    hipLaunchKernelGGL((decode_gqa_mfma_kernel<KV, false, false, false>), grid, block, 0, stream, b);
  return hipGetLastError();
}

hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, hipStream_t stream) {
  return launch_gqa_mfma<bf16_t>(a, stream);
}

hipError_t launch_decode_gqa_mfma_fp8(const DecodeArgs& a, hipStream_t stream) {
  return launch_gqa_mfma<fp8_t>(a, stream);
}

}  // namespace pa
