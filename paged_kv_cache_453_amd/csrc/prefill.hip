// Causal chunked prefill over a paged KV cache on bf16 matrix cores (MFMA).
//
// Chunked prefill splits one prompt's prefill over several rounds (xdnf.cn
// article, section 六.4); each chunk's queries sit at the last C positions of
// their sequence and must see every earlier token, the paged prefix included.
// Prefill is compute-bound (xdnf.cn article, section 六.5), so both kernels
// here are flash-attention loops on the bf16 matrix cores with fp32
// accumulation, K/V tiles gathered through the block table:
//  - bf16 caches: prefill_x32_kernel (further down), 32x32x16 products over
//    tiles staged by direct-to-LDS loads two tiles ahead;
//  - FP8 caches: prefill_mfma_kernel (first), 16x16x32 products over tiles
//    that its waves load, widen to bf16 and store to LDS.
//
// prefill_mfma_kernel.
// Tiling.  A workgroup (4 waves) owns 4*RW query rows of one head of one
// sequence; each wave owns RW rows as RW/16 blocks of 16.  Keys go in tiles of
// 64 (4 cache blocks), staged in LDS row-major (padded rows) by coalesced
// 16-byte copies: the next tile's global loads are issued before the current
// tile is computed and land in registers, and are stored to the one LDS tile
// buffer after a barrier that follows the computation (a second buffer was
// about 2% slower, and twice the LDS).  A wave skips the tiles that lie
// entirely above its causal diagonal.
//
// Orientation.  Scores are produced transposed, S^T = K Q^T, and the output as
// O^T = V^T P^T.  In a 16x16 MFMA result lane l = 16g + r holds rows 4g..4g+3
// of column r; with this orientation column = query row, so a query row's
// softmax state lives in the 4 lanes that share r, and the probabilities come
// out of the score product already laid out as the B operand of p.V (the
// reduction slots of a lane pair key groups {4g..4g+3} and {16+4g..16+4g+3} of
// a 32-key step; any order works if V uses the same one).
//  - K (A operand, key r in row r) is read from LDS with one 16-byte read per
//    lane and k-step: chunk 4ks+g of key row r.  K rows are padded by 16
//    bytes, so the 16 lanes reading one column of 16 rows hit distinct banks.
//  - V (A operand of O^T = V^T P^T, row r of d-tile t = column 16t + r) stays
//    row-major too and is read with the LDS transpose read (ds_read_b64_tr_b16):
//    in each group of 16 lanes, lane r receives element r & 3 of the 8-byte
//    pieces that lanes 4k + (r >> 2) address, k = 0..3.  So lanes 4k + q of
//    group g address columns 16t + 4q .. 16t + 4q + 3 of the key at position
//    8g + k, and lane r gets that key's column 16t + r for four keys at once;
//    two such reads give its 8 keys.  V rows are padded by 32 bytes, so the
//    eight rows of a half-wave's read cover the banks once.
//
// FP8 (E4M3) caches: the staging loads read 8 codes (8 bytes) where they would
// read 8 bf16 (16 bytes), and widen them to bf16 as they store the tile to LDS
// (exact: an E4M3 value has at most 4 significant bits); from there the
// arithmetic is that of a bf16 tile (the template also builds for bf16
// caches, which the launcher sends to the 32x32 kernel).  The per-tensor K scale is folded into the score
// scale by the caller, the V scale into the final normalisation.
//
// Softmax in base 2 with lazy rescaling: a row's reference max moves only when
// a tile's max exceeds it by more than 8, so the accumulators are rarely
// touched by the vector ALUs.  Probabilities are rounded to bf16 for the p.V
// product, and the running sum is taken over the same rounded values -- on
// the matrix cores, as the product of an all-ones operand with P^T -- so
// numerator and denominator use the same weights.  exp2 is the raw hardware
// instruction: weights below 2^-126 flush to zero, which a softmax ignores.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kKeys = 64;             // keys per tile (4 blocks)
constexpr int kEngines = 4;           // shader engines per die: a die's workgroups go to them in turn
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer resource, no format conversion
constexpr float kSlack = 8.f;         // base-2 headroom of the lazy rescale
// Starting reference max, below any score: a row that has seen only masked
// keys (a split's first tile can lie above part of a wave's diagonal) keeps
// weights exp2(-inf - kNoMax) = 0 and rescales by exp2(0) = 1, never by an
// inf - inf.
constexpr float kNoMax = -1e30f;
// bf16 1.0 in every slot: A operand whose product with P^T is the row sums
constexpr u32x4 kOnes = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS transpose read of 8 bytes (four bf16) at byte offset `off` of `base`.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* base, int off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((__attribute__((address_space(3))) const uint8_t*)base + off));
  return __builtin_bit_cast(u32x2, v);
}

// Workgroup -> (sequence, query head, query tile, key run) of a prefill launch
// of QT-row query tiles; false for a workgroup with nothing to do.
//
// How the hardware hands the workgroups out decides the order: workgroup ids
// go to the accelerator dies (XCDs, each with its own L2) round-robin, and
// within a die to its four shader engines in turn, in order -- when the next
// engine has no free slot the hand-out waits, even if the other engines have
// room.  Work per workgroup varies a lot (the causal key range grows with the
// query tile and the context; a key run past a short sequence's end is empty),
// so the ids are laid out for both:
//  * a "quad" is 4 query heads of one sequence (heads 4i .. 4i+3).  The 4
//    heads of a quad have the same key range for every (query tile, key run),
//    so every 4 consecutive ids of a die are one (query tile, key run) of the 4
//    heads of a quad: the 4 engines get equal work in lockstep and none waits
//    on another's long workgroup;
//  * quads are dealt to the dies in rounds of kXcds, every other round in
//    reverse order (die 0 takes the first and the last quad of the first two
//    rounds), so that the dies' shares of unequal sequences even out; all
//    (query tile, key run) workgroups of a quad run on its die, longer query
//    tiles first: the K/V tiles the quad stages are fetched from HBM about
//    once per die instead of once per query tile (and once for the 4 heads
//    when they share a kv head).
//  * the quads are taken sequence by sequence, the sequences in decreasing
//    order of their causal work (pairs of a query and a key it sees), so the
//    longest workgroups start first on every die instead of whenever their
//    sequence's index comes up.
// A launch has kXcds * ceil(quads / kXcds) * (query tiles x key runs) * 4 ids.
struct PrefillItem {
  int s, h, qtile, split;
};

// The sequence of rank r in decreasing order of causal work, ties by index.
// Every wave works it out from the chunk bounds and context lengths, one
// sequence per lane; batches of more than a wave of sequences keep their order.
__device__ __forceinline__ int seq_by_work(const DecodeArgs& a, int r) {
  const int n = a.num_seqs;
  if (n <= 1 || n > kWave) return r;
  const int lane = threadIdx.x & (kWave - 1);
  float work = 0.f;
  if (lane < n) {
    const int chunk = a.query_start_loc[lane + 1] - a.query_start_loc[lane];
    const int len = a.context_lens[lane];
    if (chunk > 0 && len >= chunk) work = (float)chunk * (2.f * (float)len - (float)chunk);
  }
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, work), j));
    rank += (wj > work) || (wj == work && j < lane);
  }
  const uint64_t hit = __ballot(lane < n && rank == r);
  return hit != 0 ? (int)__builtin_ctzll(hit) : r;
}
__device__ __forceinline__ bool prefill_item(const DecodeArgs& a, int QT, PrefillItem& it) {
  const int nsplit_max = a.partition_blocks > 0 ? a.max_partitions : 1;
  const int qt_count = (a.max_query_len + QT - 1) / QT;
  const int X = qt_count * nsplit_max;               // (query tile, key run) members
  const int quads_per_seq = (a.num_heads + kEngines - 1) / kEngines;
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;                  // position on the die
  const int round = k / (X * kEngines);
  const int rem = k - round * (X * kEngines);
  const int member = rem / kEngines;
  const int quad = round * kXcds + ((round & 1) ? kXcds - 1 - xcd : xcd);
  if (quad >= a.num_seqs * quads_per_seq) return false;
  const int rank = quad / quads_per_seq;
  it.s = seq_by_work(a, rank);
  it.h = (quad - rank * quads_per_seq) * kEngines + (rem - member * kEngines);
  if (it.h >= a.num_heads) return false;
  it.qtile = qt_count - 1 - member / nsplit_max;     // later (longer) tiles first
  it.split = member % nsplit_max;
  return true;
}

}  // namespace

template <typename KV, int D, int RW, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_mfma_kernel(DecodeArgs a) {
  constexpr bool kFp8 = sizeof(KV) == 1;
  constexpr int KS = D / 32;            // k-steps of the score MFMA
  constexpr int DT = D / 16;            // d-tiles of the output (= columns per lane per key)
  constexpr int QB = RW / 16;           // 16-row query blocks per wave
  constexpr int QT = NW * RW;           // query rows per workgroup (NW waves)
  constexpr int NT = 64 * NW;           // threads per workgroup
  constexpr int ROW = D * 2 + 16;       // padded LDS row of K, bytes
  constexpr int ROWV = D * 2 + 32;      // padded LDS row of V, bytes
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int KPP = NT / CH;          // key rows staged per pass of the workgroup
  constexpr int NPASS = kKeys / KPP;    // staging passes per tile
  constexpr int TILE = kKeys * (ROW + ROWV);   // K rows, then V rows
  __shared__ __attribute__((aligned(16))) uint8_t smem[TILE];
  __shared__ int sh_bad;

  // with split-K (a.partition_blocks > 0) the causal key range of a query
  // tile is cut into runs of a.partition_blocks blocks, one workgroup each
  PrefillItem it;
  if (!prefill_item(a, QT, it)) return;
  const int s = it.s, h = it.h, qtile = it.qtile, split = it.split;
  const int nsplit_max = a.partition_blocks > 0 ? a.max_partitions : 1;
  const int qt_count = (a.max_query_len + QT - 1) / QT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_uniform(tid >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int hq = a.num_heads;
  const int kvh = h / a.group;

  const int q0 = a.query_start_loc[s];
  const int q1 = a.query_start_loc[s + 1];
  // rows outside [0, num_query_tokens) cannot be written at all
  if (q0 < 0 || q1 < q0 || q1 > a.num_items) return;
  const int chunk = q1 - q0;
  const int len = a.context_lens[s];
  const int qr0 = qtile * QT;
  if (qr0 >= chunk) return;
  // (with split-K the workspace holds the splits of max_context_len keys)
  const bool bad = chunk > len || chunk > a.max_query_len || len > a.max_blocks_per_seq * kBlock ||
                   (a.partition_blocks > 0 && len > a.max_context_len);
  const int prefix = len - chunk;
  bf16_t* out = static_cast<bf16_t*>(a.out);

  if (bad) {
    // the whole chunk of this sequence is reported as NaN (by the first split;
    // the merge leaves such rows alone).  The grid has tiles for max_query_len
    // rows only, so a longer chunk is covered by striding over them.
    if (split != 0) return;
    for (int base = qr0; base < chunk; base += qt_count * QT)
      for (int i = tid; i < QT * D; i += NT) {
        const int rr = base + i / D;
        if (rr < chunk) out[((int64_t)(q0 + rr) * hq + h) * D + i % D] = 0x7FC0;
      }
    return;
  }
  if (tid == 0) sh_bad = 0;
  lds_barrier();

  // this wave's query rows: qw0 .. qw0+RW-1 (chunk-relative), positions prefix + row
  const int qw0 = qr0 + w * RW;
  const int wave_rows = max(0, min(RW, chunk - qw0));
  const int wave_first_pos = prefix + qw0;
  const int wave_last_pos = prefix + qw0 + wave_rows - 1;

  const int qlast = min(chunk, qr0 + QT) - 1;
  const int kend = prefix + qlast + 1;            // keys [0, kend) matter to this workgroup
  const int ntiles = (kend + kKeys - 1) / kKeys;
  const int nblk = (kend + kBlock - 1) / kBlock;
  const int split_tiles = a.partition_blocks > 0 ? a.partition_blocks / 4 : ntiles;
  const int nsplit = a.partition_blocks > 0 ? (ntiles + split_tiles - 1) / split_tiles : 1;
  if (split >= nsplit) return;   // the whole workgroup: no barrier is left waiting

  // Q^T as the B operand: lane (r, g) holds chunk 4ks+g of query row 16qb + r.
  u32x4 qop[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + 16 * qb + r;
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.query) + ((int64_t)(q0 + qi) * hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[qb][ks] = qi < chunk ? *reinterpret_cast<const u32x4*>(qsrc + 8 * (4 * ks + g))
                               : u32x4{0u, 0u, 0u, 0u};
  }

  const float sl2 = a.scale_log2;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const KV* kpool = static_cast<const KV*>(a.k_cache);
  const KV* vpool = static_cast<const KV*>(a.v_cache);

  // Staging: thread (key row kr0 + KPP*p, chunk cc) for p < NPASS.  Block ids
  // of a tile sit in lanes 0..3 of ids, repeated across the wave (fetched two
  // tiles ahead from an in-bounds, clamped index).  Each lane works out, on
  // the vector ALUs and once per tile, the pool offset and live bytes of
  // block lane & 3; every pass then reads its block's pair into scalars.  The
  // rows of one pass of one wave lie in one block.  Each block is read
  // through a buffer resource sized to its live rows (keys < kend), so rows
  // past the end, blocks past the last one and ids outside the pool read as
  // zeros without touching memory.  All staging loads are unconditional,
  // which keeps the compiler's load counting exact: the waits before the LDS
  // stores cover only what they store.
  static_assert(kKeys == 4 * kBlock && KPP % kBlock == 0 && (64 / CH) <= kBlock,
                "a pass of a wave stays in one block");
  const int cc = tid % CH;
  const int kr0 = tid / CH;
  const int row_bytes = D * (int)sizeof(KV);
  // the byte of its row a thread loads, the same in every pass (KPP rows apart)
  const int lane_off = (kr0 % kBlock) * row_bytes + cc * 8 * (int)sizeof(KV);
  // what one thread loads per key row: 8 elements (16 bytes of bf16, 8 of fp8)
  typedef typename std::conditional<kFp8, u32x2, u32x4>::type piece_t;
  const auto fetch_ids = [&](int kt) {
    const int j = kt * 4 + (lane & 3);
    return table[min(j, a.max_blocks_per_seq - 1)];
  };
  piece_t kst[NPASS], vst[NPASS];
  const auto stage_load = [&](int kt, int ids) {
    const int gb = kt * 4 + (lane & 3);                     // block within the sequence
    const bool in_pool = ids >= 0 && (int64_t)ids < a.num_blocks;
    const int rows = gb < nblk ? min(kBlock, kend - gb * kBlock) : 0;
    if (rows > 0 && !in_pool) sh_bad = 1;
    const bool live = rows > 0 && in_pool;
    const int64_t off =
        live ? ((int64_t)ids * a.num_kv_heads + kvh) * (kBlock * D * (int)sizeof(KV)) : 0;
    const int nbytes = live ? rows * row_bytes : 0;
    const uint32_t off_lo = (uint32_t)off, off_hi = (uint32_t)((uint64_t)off >> 32);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int bt = (KPP * p + (64 / CH) * w) / kBlock;   // this wave's block in the tile
      const uint64_t boff =
          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_hi, bt) << 32) |
          (uint32_t)__builtin_amdgcn_readlane((int)off_lo, bt);
      const int nb = __builtin_amdgcn_readlane(nbytes, bt);
      const auto krs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(kpool) + boff), 0, nb, kBufferWord3);
      const auto vrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(vpool) + boff), 0, nb, kBufferWord3);
      if constexpr (kFp8) {
        kst[p] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(krs, lane_off, 0, 0));
        vst[p] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, lane_off, 0, 0));
      } else {
        kst[p] = __builtin_amdgcn_raw_buffer_load_b128(krs, lane_off, 0, 0);
        vst[p] = __builtin_amdgcn_raw_buffer_load_b128(vrs, lane_off, 0, 0);
      }
    }
  };
  const auto widen = [](const piece_t& x) -> u32x4 {
    if constexpr (kFp8) {
      const u32x2 lo = fp8x4_to_bf16x4(x[0]), hi = fp8x4_to_bf16x4(x[1]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      return x;
    }
  };
  const auto stage_store = [&]() {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int kr = kr0 + KPP * p;
      *reinterpret_cast<u32x4*>(&smem[kr * ROW + cc * 16]) = widen(kst[p]);
      *reinterpret_cast<u32x4*>(&smem[kKeys * ROW + kr * ROWV + cc * 16]) = widen(vst[p]);
    }
  };

  f32x4 o[QB][DT];
  f32x4 lacc[QB];      // every element: the row's running sum of weights
  float mref[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mref[qb] = kNoMax;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DT; ++t) o[qb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // this workgroup's key tiles [kt0, kt1); a prefetch past kt1 asks for tile
  // ntiles, past the end, which reads nothing
  const int kt0 = split * split_tiles;
  const int kt1 = min(ntiles, kt0 + split_tiles);
  const auto in_range = [&](int kt) { return kt < kt1 ? kt : ntiles; };
  int ids_next = fetch_ids(kt0);
  stage_load(kt0, ids_next);
  ids_next = fetch_ids(in_range(kt0 + 1));
  stage_store();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int ids_cur = ids_next;
    stage_load(in_range(kt + 1), ids_cur);   // past the last tile: empty resources, no traffic
    ids_next = fetch_ids(in_range(kt + 2));
    lds_barrier();   // tile kt is in the buffer

    const int tile_first = kt * kKeys;
    if (wave_rows > 0 && tile_first <= wave_last_pos) {
      const uint8_t* kb = smem;
      const uint8_t* vb = smem + kKeys * ROW;
      const bool need_mask = tile_first + kKeys - 1 > wave_first_pos;

      // ---- S^T = K Q^T: four 16-key groups ----
      f32x4 sc[QB][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        u32x4 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[ks] = *reinterpret_cast<const u32x4*>(kb + (16 * nt + r) * ROW + 16 * (4 * ks + g));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sc[qb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sc[qb][nt] = mfma_16x16x32(ka[ks], qop[qb][ks], sc[qb][nt]);
        }
      }

      // ---- online softmax; lane holds S[row 16qb + r][key tile_first + 16nt + 4g + i] ----
      // The common path needs no cross-lane step: each lane checks its own
      // max against the row's reference, and only if some lane of the wave
      // exceeds it by more than kSlack is the row max gathered and the
      // reference moved (rare after the first tile).
      u32x4 pk[2][QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = wave_first_pos + 16 * qb + r;
        if (need_mask) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[qb][nt][i] = (tile_first + 16 * nt + 4 * g + i <= qpos) ? sc[qb][nt][i] : -INFINITY;
        }
        float lmax = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          lmax = fmaxf(lmax, fmaxf(fmaxf(sc[qb][nt][0], sc[qb][nt][1]),
                                   fmaxf(sc[qb][nt][2], sc[qb][nt][3])));
        lmax *= sl2;
        if (__ballot(lmax > mref[qb] + kSlack) != 0) {
          float rmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
          rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));
          const float mn = rmax > mref[qb] + kSlack ? rmax : mref[qb];
          const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mn);
          lacc[qb] *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t) o[qb][t] *= alpha;
          mref[qb] = mn;
        }
        const float nmr = -mref[qb];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t wv[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const f32x4& sv = sc[qb][2 * kk + x / 2];
            const int i0 = 2 * (x % 2);
            wv[x] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[i0], sl2, nmr)),
                                __builtin_amdgcn_exp2f(fmaf(sv[i0 + 1], sl2, nmr)));
          }
          pk[kk][qb] = u32x4{wv[0], wv[1], wv[2], wv[3]};
          // row sum of the rounded weights on the matrix cores: all-ones A operand
          lacc[qb] = mfma_16x16x32(kOnes, pk[kk][qb], lacc[qb]);
        }
      }

      // ---- O^T += V^T P^T, 32 keys per step ----
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // positions 8g + k (k < 4) hold key 4g + k of the step, 8g + 4 + k key
        // 16 + 4g + k, as in the weights' operand
        const int vrow = 32 * kk + 4 * g + ((lane & 15) >> 2);
        const int vcol = 2 * 4 * (lane & 3);
        u32x4 va[DT];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const u32x2 lo = lds_read_tr16(vb, vrow * ROWV + 32 * t + vcol);
          const u32x2 hi = lds_read_tr16(vb, (vrow + 16) * ROWV + 32 * t + vcol);
          va[t] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][t] = mfma_16x16x32(va[t], pk[kk][qb], o[qb][t]);
      }
    }
    lds_barrier();   // every wave is done with tile kt
    stage_store();
  }

  // ---- normalise and store: lane holds O[row 16qb + r][16t + 4g + i] ----
  lds_barrier();
  const bool poisoned = sh_bad != 0;
  if (nsplit > 1) {
    // a split's partial: its normalised output and the natural-log sum of
    // exp(scores) over its keys; a row that saw none of them weighs nothing
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = lacc[qb][0];
      const int qi = qw0 + 16 * qb + r;
      if (qi >= chunk) continue;
      const float inv = l > 0.f ? (kFp8 ? a.v_scale : 1.f) / l : 0.f;
      const int64_t row = ((int64_t)(q0 + qi) * hq + h) * nsplit_max + split;
      float* dst = a.part_o + row * D;
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < DT; ++t)
        *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * g) =
            poisoned ? f32x4{nan, nan, nan, nan} : o[qb][t] * inv;
      if (g == 0)
        a.part_lse[row] = poisoned ? nan : l > 0.f ? (mref[qb] + log2f(l)) * kLn2 : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = lacc[qb][0];
    const int qi = qw0 + 16 * qb + r;
    if (qi >= chunk) continue;
    const float inv = (kFp8 ? a.v_scale : 1.f) / l;
    bf16_t* dst = out + ((int64_t)(q0 + qi) * hq + h) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const uint32_t lo = poisoned ? 0x7FC07FC0u : pack_bf16x2(o[qb][t][0] * inv, o[qb][t][1] * inv);
      const uint32_t hi = poisoned ? 0x7FC07FC0u : pack_bf16x2(o[qb][t][2] * inv, o[qb][t][3] * inv);
      *reinterpret_cast<u32x2*>(dst + 16 * t + 4 * g) = u32x2{lo, hi};
    }
  }
}

// Direct-to-LDS, software-pipelined prefill for bf16 caches on 32x32 products.
//
// Staging.  Each wave copies one of the tile's four cache blocks (its K and V
// slabs) with direct-to-LDS buffer loads: one instruction moves 1 KB, 64 lanes
// x 16 bytes written to consecutive LDS addresses, so no register holds the
// tile on its way and no LDS store instruction is issued.  Each block goes
// through a buffer resource sized to its live rows: rows past the end, blocks
// past the last one and ids outside the pool are written as zeros (checked on
// the part).  Rows are not padded (the loads write contiguous LDS); instead a
// lane loads the global 16-byte chunk that its LDS position should hold under
// an XOR swizzle, chosen from bank-conflict counters measured on the part:
//  - K (read as 16-byte A operands, 16 rows x one chunk per group of lanes):
//    LDS chunk p of row r holds chunk p ^ (r mod 16) (D = 128), p ^ ((r / 2)
//    mod 8) (D = 64);
//  - V (read with the transposing 8-byte LDS read, 8 rows x 64 bytes per
//    instruction): chunk p of row r holds chunk p ^ 4 (r mod 4) (D = 128),
//    p ^ 4 ((r / 2) mod 2) (D = 64).
// K and V each have two tile buffers (64 KB in all at D = 128, so two
// workgroups fit a compute unit).
//
// Pipeline.  K runs one tile ahead of V: during iteration kt the LDS holds K
// of tile kt+1 and V of tile kt, and the loads of K of kt+2 and V of kt+1 --
// issued at the top of the iteration into the buffers the previous iteration
// finished with -- are in flight.  A wave holds the scores of tile kt, masked
// and with their max taken in the previous iteration, and computes: the lazy
// reference-max check of tile kt (a rescale is rare), then the score MFMAs of
// tile kt+1 interleaved with exp2 and the bf16 packing of tile kt's weights,
// then the row sums (v_dot2c of the packed weights with ones) and p.V MFMAs of
// tile kt, then the causal mask and row maxima of tile kt+1.  One barrier per
// tile, after each wave has waited for its own loads.  The arithmetic of every
// (query, key) pair is that of prefill_mfma_kernel.
template <int D> __device__ __forceinline__ int k_swizzle(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// V rows for the 32x32 products' transposed reads (8 rows x 64 bytes per
// instruction): chunk p of row `row` is stored at chunk p ^ v32_swizzle(row).
template <int D> __device__ __forceinline__ int v32_swizzle(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma_32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One direct-to-LDS load: 64 lanes x 16 bytes from buffer `rs` at the lanes'
// byte offsets `voff`, written to the 1 KB of LDS at `lds` (lane i at lds + 16 i).
// POLICY: cache-policy bits, 0 or 2 (nontemporal: the lines are evicted first).
template <int POLICY>
__device__ __forceinline__ void load_lds_1k(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, POLICY);
}

// max(a, b, c) in one instruction, with fmaxf's rule for NaN operands (they
// are ignored).  Written out because for fmaxf of matrix-core results the
// compiler first quiets each operand with an extra max of it with itself.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// Orders this wave's memory accesses around a workgroup barrier without the
// waits a memory fence implies: the loads into the next tile buffers must stay
// in flight across it.
__device__ __forceinline__ void plain_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// The products.  v_mfma_f32_32x32x16_bf16 (32 x 32 results, 16-deep k-steps)
// runs at nearly the part's bf16 peak in a loop of independent products, where
// the 16x16x32 form reaches little more than half of it.  Lane l = 32 hh + r
// supplies row r of the A operand and column r of the B operand, k-slots
// 8 hh .. 8 hh + 7 of each k-step, and holds result rows 8 i + 4 hh + j
// (j < 4) of column r in result register 4 i + j.  A wave owns 32 query rows,
// the columns of both products:
//  - scores S^T = K Q^T: A is 32 keys of the K tile (16-byte swizzled reads),
//    B is the wave's Q, held in registers for the whole walk;
//  - O^T += V^T P^T: step (kb, p) takes keys 32 kb + 16 p + {4 hh + (0..3),
//    8 + 4 hh + (0..3)} in lane (hh, r), exactly that lane's own scores
//    8 p .. 8 p + 7 of key block kb, so the weights need no data movement; A
//    is 32 dims of those keys from two transposing 8-byte LDS reads.
// A row's 64 scores of a tile sit in two lanes (r and r + 32), 32 each; its
// max and sum combine the two with one cross-lane step.

// STREAM: K/V tiles loaded with the nontemporal hint, for launches in which no
// other workgroup reads them (see the launcher).
template <int D, int NW, bool STREAM>
__global__ __launch_bounds__(64 * NW, 2) void prefill_x32_kernel(DecodeArgs a) {
  static_assert(NW == 4, "one wave per cache block of a 64-key tile");
  constexpr int RW = 32;                // query rows per wave: the 32 columns of the products
  constexpr int KS = D / 16;            // k-steps of the score MFMA (16 dims each)
  constexpr int DB = D / 32;            // 32-dim blocks of the output
  constexpr int QT = NW * RW;           // query rows per workgroup
  constexpr int NT = 64 * NW;           // threads per workgroup
  constexpr int RB = D * 2;             // bytes per K or V row
  constexpr int TILE = kKeys * RB;      // bytes per K or V tile
  constexpr int SLAB = kBlock * RB;     // bytes per (block, kv head) slab
  constexpr int NLD = SLAB / 1024;      // 1 KB loads per slab
  constexpr int RPL = 1024 / RB;        // rows per 1 KB load
  // four separate LDS objects, so that the compiler's wait for loads into one
  // buffer is not imposed on reads of the other
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[TILE];
  __shared__ int sh_bad;

  PrefillItem it;
  if (!prefill_item(a, QT, it)) return;
  const int s = it.s, h = it.h, qtile = it.qtile, split = it.split;
  const int nsplit_max = a.partition_blocks > 0 ? a.max_partitions : 1;
  const int qt_count = (a.max_query_len + QT - 1) / QT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_uniform(tid >> 6);
  const int r = lane & 31;              // this lane's query row (column of the products)
  const int hh = lane >> 5;             // which half of each k-step it supplies
  const int hq = a.num_heads;
  const int kvh = h / a.group;

  const int q0 = a.query_start_loc[s];
  const int q1 = a.query_start_loc[s + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.num_items) return;
  const int chunk = q1 - q0;
  const int len = a.context_lens[s];
  const int qr0 = qtile * QT;
  if (qr0 >= chunk) return;
  const bool bad = chunk > len || chunk > a.max_query_len || len > a.max_blocks_per_seq * kBlock ||
                   (a.partition_blocks > 0 && len > a.max_context_len);
  const int prefix = len - chunk;
  bf16_t* out = static_cast<bf16_t*>(a.out);

  if (bad) {
    if (split != 0) return;
    for (int base = qr0; base < chunk; base += qt_count * QT)
      for (int i = tid; i < QT * D; i += NT) {
        const int rr = base + i / D;
        if (rr < chunk) out[((int64_t)(q0 + rr) * hq + h) * D + i % D] = 0x7FC0;
      }
    return;
  }
  const int qw0 = qr0 + w * RW;
  const int wave_rows = max(0, min(RW, chunk - qw0));
  const int wave_first_pos = prefix + qw0;
  const int wave_last_pos = prefix + qw0 + wave_rows - 1;

  const int qlast = min(chunk, qr0 + QT) - 1;
  const int kend = prefix + qlast + 1;
  const int ntiles = (kend + kKeys - 1) / kKeys;
  const int nblk = (kend + kBlock - 1) / kBlock;
  const int split_tiles = a.partition_blocks > 0 ? a.partition_blocks / 4 : ntiles;
  const int nsplit = a.partition_blocks > 0 ? (ntiles + split_tiles - 1) / split_tiles : 1;
  if (split >= nsplit) return;   // the whole workgroup: no barrier is left waiting
  const int kt0 = split * split_tiles;
  const int kt1 = min(ntiles, kt0 + split_tiles);
  // tiles this wave sees any key of: kt0 .. wave_end-1; from mask_from on, a
  // tile holds keys past some of its rows (the causal diagonal, and the
  // zero-filled rows past kend), masked before the tile's max is taken
  const int wave_end = wave_rows > 0 ? max(kt0, min(kt1, wave_last_pos / kKeys + 1)) : kt0;
  const int mask_from = (wave_first_pos + 1) / kKeys;
  if (tid == 0) sh_bad = 0;
  plain_barrier();   // before any staging can set it

  // Q^T as the B operand: lane (hh, r) holds dims 16 ks + 8 hh .. +7 of query row r
  u32x4 qop[KS];
  {
    const int qi = qw0 + r;
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.query) + ((int64_t)(q0 + qi) * hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = qi < chunk ? *reinterpret_cast<const u32x4*>(qsrc + 8 * (2 * ks + hh))
                           : u32x4{0u, 0u, 0u, 0u};
  }

  const float sl2 = a.scale_log2;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_cache);

  // Byte offsets inside a slab that lane `lane` loads for load j: its LDS row
  // (tile row 16 w + RPL j + lane / (RB / 16)) and the swizzled chunk there.
  int koff[NLD], voff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int row = RPL * j + lane / (RB / 16);    // row in the slab = tile row mod 16
    const int p = lane % (RB / 16);
    koff[j] = row * RB + 16 * (p ^ k_swizzle<D>(row));
    voff[j] = row * RB + 16 * (p ^ v32_swizzle<D>(row));
  }
  // This wave's block of tile kt: its id, read through the constant address
  // space (the table is not written during the call) so that it is a scalar
  // load, counted apart from the vector loads into the tile buffers.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* ctable = (const_i32*)table;
  const auto block_id = [&](int kt) { return ctable[min(kt * 4 + w, a.max_blocks_per_seq - 1)]; };
  // This wave's slab of tile kt (block id `id`): its byte offset in a pool and
  // its live bytes (0: past the keys, or an id outside the pool, which
  // poisons the workgroup's rows).  The K and V slabs of a tile share it.
  struct Slab {
    int64_t off;
    int bytes;
  };
  const uint32_t pool_ids = (uint32_t)min<int64_t>(a.num_blocks, 0x80000000ll);
  const int64_t id_stride = (int64_t)a.num_kv_heads * SLAB;
  const int64_t head_off = (int64_t)kvh * SLAB;
  int bad_id = 0;        // this wave staged a block id outside the pool
  const auto describe = [&](int kt, int id) {
    const int gb = kt * 4 + w;
    const int rows = gb < nblk ? min(kBlock, kend - gb * kBlock) : 0;
    const bool in_pool = (uint32_t)id < pool_ids;
    bad_id |= (int)(rows > 0) & (int)!in_pool;
    const bool live = rows > 0 && in_pool;
    return Slab{live ? id * id_stride + head_off : 0, live ? rows * RB : 0};
  };
  const auto stage = [&](uint8_t* dst_base, const uint8_t* pool, const int (&off)[NLD],
                         const Slab& sl) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pool + sl.off), 0,
                                                      sl.bytes, kBufferWord3);
#pragma unroll
    for (int j = 0; j < NLD; ++j)
      load_lds_1k<STREAM ? 2 : 0>(rs, dst_base + w * SLAB + j * 1024, off[j]);
  };
  // every load of this wave has landed and no LDS read is outstanding; then
  // meet the other waves
  const auto sync_tiles = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    plain_barrier();
  };

  // O^T: o[db][4i + j] is dim 32 db + 8 i + 4 hh + j of query row r
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float lsum = 0.f;      // this lane's half of the row's sum of weights
  float mref = kNoMax;   // the row's reference max (base 2), the same in both its lanes

  // S^T = K Q^T from a K buffer: sc[kb][4i + j] is key 32 kb + 8 i + 4 hh + j of row r
  const auto scores = [&](const uint8_t* kbuf, f32x16 (&sc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * kb + r;
      sc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(
            kbuf + row * RB + 16 * ((2 * ks + hh) ^ k_swizzle<D>(row)));
        sc[kb] = mfma_32x32x16(ka, qop[ks], sc[kb]);
      }
    }
  };
  // max of the lane's 32 scores of a tile, in base 2 (masked keys are -inf):
  // a tree of three-way maxes
  const auto row_max = [&](const f32x16 (&sc)[2], float& lmax) {
    float m1[11];
#pragma unroll
    for (int x = 0; x < 10; ++x) {
      const int e = 3 * x;
      m1[x] = max3f(sc[e / 16][e % 16], sc[(e + 1) / 16][(e + 1) % 16],
                    sc[(e + 2) / 16][(e + 2) % 16]);
    }
    m1[10] = fmaxf(sc[1][14], sc[1][15]);
    const float a = max3f(m1[0], m1[1], m1[2]);
    const float b = max3f(m1[3], m1[4], m1[5]);
    const float c = max3f(m1[6], m1[7], m1[8]);
    lmax = max3f(max3f(a, b, c), m1[9], m1[10]) * sl2;
  };
  // causal mask of tile kt: keys past a row's position get -inf
  const auto mask = [&](f32x16 (&sc)[2], int kt) {
    const int rel = wave_first_pos + r - kt * kKeys - 4 * hh;   // key index limit, tile-relative
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        sc[kb][q] = (32 * kb + 8 * (q / 4) + (q % 4) <= rel) ? sc[kb][q] : -INFINITY;
  };
  // lazy reference-max check against a tile's visible max (rare rescale)
  const auto rescale = [&](float lmax) {
    if (__ballot(lmax > mref + kSlack) != 0) {
      const float rmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
      const float mn = rmax > mref + kSlack ? rmax : mref;
      const float alpha = __builtin_amdgcn_exp2f(mref - mn);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      mref = mn;
    }
  };
  // P^T as the B operand of the p.V steps: step (kb, p) covers keys
  // 32 kb + 16 p + {0..15}; lane (hh, r) supplies keys 4 hh + {0..3} and
  // 8 + 4 hh + {0..3} of it, which are its own scores sc[kb][8p .. 8p+7]
  const auto weights = [&](const f32x16 (&sc)[2], u32x4 (&pk)[2][2]) {
    const float nmr = -mref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t wv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          wv[x] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[kb][8 * p + 2 * x], sl2, nmr)),
                              __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * p + 2 * x + 1], sl2, nmr)));
        pk[kb][p] = u32x4{wv[0], wv[1], wv[2], wv[3]};
      }
  };
  // row sums of the bf16 weights (the values the products use), and
  // O^T += V^T P^T from a V buffer: the A operand of step (kb, p), d-block db
  // is dims 32 db + r of those keys, two transposed 8-byte reads per lane
  const auto accumulate = [&](const uint8_t* vbuf, const u32x4 (&pk)[2][2]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          // (a named copy: a bit_cast of the vector element itself compiled to
          // element 0 for every x)
          const uint32_t pair = pk[kb][p][x];
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, lsum, false);
        }
    const int t = lane & 15;
    const int c0 = 16 * ((lane >> 4) & 1) + 4 * (t & 3);   // this lane's first column in a d-block
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int row = 32 * kb + 16 * p + 4 * hh + (t >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int b = 2 * (32 * db + c0);
          const u32x2 lo = lds_read_tr16(
              vbuf, row * RB + 16 * ((b >> 4) ^ v32_swizzle<D>(row)) + (b & 15));
          const u32x2 hi = lds_read_tr16(
              vbuf, (row + 8) * RB + 16 * ((b >> 4) ^ v32_swizzle<D>(row + 8)) + (b & 15));
          o[db] = mfma_32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk[kb][p], o[db]);
        }
      }
  };

  const auto in_range = [&](int kt) { return kt < kt1 ? kt : ntiles; };

  // prologue: K of kt0 and kt0+1, V of kt0; the scores of tile kt0
  f32x16 sa[2], sb[2];
  float lm = 0.f;
  int id_k = block_id(in_range(kt0 + 2));   // K of kt+2, staged in iteration kt
  Slab slab_v;                              // V of kt+1: the slab its K was staged from
  {
    const Slab s0 = describe(kt0, block_id(kt0));
    slab_v = describe(in_range(kt0 + 1), block_id(in_range(kt0 + 1)));
    stage(kbuf0, kpool, koff, s0);
    stage(vbuf0, vpool, voff, s0);
    stage(kbuf1, kpool, koff, slab_v);
    sync_tiles();
    if (kt0 < wave_end) {
      scores(kbuf0, sa);
      if (kt0 >= mask_from) mask(sa, kt0);
      row_max(sa, lm);
    }
    sync_tiles();
  }

  // iteration kt, with P = (kt - kt0) mod 2: K of kt+1 is in kbuf(1-P), V of kt
  // in vbuf(P); K of kt+2 goes to kbuf(P), V of kt+1 to vbuf(1-P)
  const auto iteration = [&](auto parity, int kt, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    constexpr int P = decltype(parity)::value;
    uint8_t* const k_now = P ? kbuf0 : kbuf1;    // K of kt+1
    uint8_t* const k_next = P ? kbuf1 : kbuf0;   // K of kt+2
    uint8_t* const v_now = P ? vbuf1 : vbuf0;    // V of kt
    uint8_t* const v_next = P ? vbuf0 : vbuf1;   // V of kt+1
    const Slab slab_k = describe(in_range(kt + 2), id_k);
    stage(k_next, kpool, koff, slab_k);
    stage(v_next, vpool, voff, slab_v);
    slab_v = slab_k;
    id_k = block_id(in_range(kt + 3));
    if (kt < wave_end) {
      // cur holds tile kt's scores, masked where needed, and lm their max
      rescale(lm);
      // The next tile's scores are computed even past the wave's last tile
      // (then from zeros or keys it does not see, never used), so that each
      // phase is one straight block whose matrix and vector work can be
      // interleaved.
      // (the compiler's own interleaving of the two: fixed orders of reads,
      // products and vector work measured 2-5% slower)
      u32x4 pk[2][2];
      scores(k_now, nxt);
      weights(cur, pk);
      accumulate(v_now, pk);
      // the next tile's max over the keys its rows see
      if (__builtin_expect(kt + 1 >= mask_from && kt + 1 < wave_end, 0)) mask(nxt, kt + 1);
      row_max(nxt, lm);
    }
    sync_tiles();
  };
  for (int kt = kt0; kt < kt1; kt += 2) {
    iteration(std::integral_constant<int, 0>(), kt, sa, sb);
    if (kt + 1 >= kt1) break;
    iteration(std::integral_constant<int, 1>(), kt + 1, sb, sa);
  }

  // a wave that staged an id outside the pool poisons the workgroup's rows
  if (bad_id) sh_bad = 1;
  sync_tiles();
  const bool poisoned = sh_bad != 0;
  const float l = lsum + __shfl_xor(lsum, 32, 64);
  const int qi = qw0 + r;
  if (nsplit > 1) {
    if (qi >= chunk) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t row = ((int64_t)(q0 + qi) * hq + h) * nsplit_max + split;
    float* dst = a.part_o + row * D;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * i + 4 * hh) =
            poisoned ? f32x4{nan, nan, nan, nan}
                     : f32x4{o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                             o[db][4 * i + 3] * inv};
    if (hh == 0)
      a.part_lse[row] = poisoned ? nan : l > 0.f ? (mref + log2f(l)) * kLn2 : -INFINITY;
    return;
  }
  if (qi >= chunk) return;
  const float inv = 1.f / l;
  bf16_t* dst = out + ((int64_t)(q0 + qi) * hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = poisoned ? 0x7FC07FC0u
                                   : pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
      const uint32_t hi = poisoned ? 0x7FC07FC0u
                                   : pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
      *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * i + 4 * hh) = u32x2{lo, hi};
    }
}

// 32 query rows per wave: each K/V operand read from LDS feeds two 16-row
// blocks (16 rows per wave measured 15% slower on the mixed workload's chunks).
constexpr int kPrefillRowsPerWave = 32;
// waves per workgroup: they share each staged K/V tile.  8 waves (256 query
// rows) stage half as much per row but measured mixed: 3% faster on 256-row
// chunks over cached prefixes, 7% on long unsplit prefixes, 16% slower on
// grouped-query chunks and 9% slower split over keys.
constexpr int kPrefillWaves = 4;

// Merge of a split query tile's partials: for each of its rows,
// out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M) with M = max_p lse_p
// (exact in real arithmetic), the split-K rule of decode applied to the key
// runs of a prefill tile.  One workgroup per (quarter of a query tile, head,
// sequence): it finds the tile's number of splits as the prefill kernel did
// and returns at once for an unsplit tile or a sequence that broke the
// contract (its NaN is already written).  Threads first take one row each for
// M and the sum of weights (LDS), then pieces of 8 columns of the rows, whose
// partial loads are independent of each other.
constexpr int kMergeParts = 4;          // workgroups per query tile
template <int D, int QT>
__global__ __launch_bounds__(256) void prefill_merge_kernel(DecodeArgs a) {
  constexpr int CW = 8;                 // columns per piece
  constexpr int QR = QT / kMergeParts;  // rows of this workgroup
  constexpr int NPIECE = QR * (D / CW);
  __shared__ float sh_m[QR];
  __shared__ float sh_inv[QR];
  const int qtile = blockIdx.x / kMergeParts;
  const int quarter = blockIdx.x % kMergeParts;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int q0 = a.query_start_loc[s];
  const int q1 = a.query_start_loc[s + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.num_items) return;
  const int chunk = q1 - q0;
  const int len = a.context_lens[s];
  const int qr0 = qtile * QT;
  if (qr0 >= chunk) return;
  if (chunk > len || chunk > a.max_query_len || len > a.max_blocks_per_seq * kBlock ||
      len > a.max_context_len)
    return;
  const int kend = len - chunk + min(chunk, qr0 + QT);
  const int ntiles = (kend + kKeys - 1) / kKeys;
  const int split_tiles = a.partition_blocks / 4;
  const int n = (ntiles + split_tiles - 1) / split_tiles;
  if (n <= 1) return;
  const int r0 = qr0 + quarter * QR;   // first chunk row of this workgroup
  const int rows = min(QR, chunk - r0);
  if (rows <= 0) return;
  const int hq = a.num_heads;
  const int P = a.max_partitions;
  const auto row_base = [&](int rr) { return ((int64_t)(q0 + r0 + rr) * hq + h) * P; };
  for (int rr = threadIdx.x; rr < QR; rr += blockDim.x) {
    float mm = -INFINITY, sum = 0.f;
    bool nan = false;
    if (rr < rows) {
      const float* lse = a.part_lse + row_base(rr);
      for (int p = 0; p < n; ++p) {
        const float x = lse[p];
        nan |= isnan(x);
        mm = fmaxf(mm, x);
      }
      for (int p = 0; p < n; ++p) sum += expf(lse[p] - mm);
    }
    sh_m[rr] = mm;
    sh_inv[rr] = nan ? __builtin_nanf("") : 1.f / sum;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NPIECE; i += blockDim.x) {
    const int rr = i / (D / CW);
    if (rr >= rows) break;
    const int c = (i - rr * (D / CW)) * CW;
    const int64_t base = row_base(rr);
    const float mm = sh_m[rr];
    float acc[CW];
#pragma unroll
    for (int e = 0; e < CW; ++e) acc[e] = 0.f;
    for (int p = 0; p < n; ++p) {
      const float wt = expf(a.part_lse[base + p] - mm);
      const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + (base + p) * D + c);
      const f32x4 lo = src[0], hi = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(wt, lo[e], acc[e]);
        acc[4 + e] = fmaf(wt, hi[e], acc[4 + e]);
      }
    }
    const float inv = sh_inv[rr];
    u32x4 wv;
#pragma unroll
    for (int x = 0; x < 4; ++x) wv[x] = pack_bf16x2(acc[2 * x] * inv, acc[2 * x + 1] * inv);
    *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.out) + (int64_t)(q0 + r0 + rr) * hq * D +
                              (int64_t)h * D + c) = wv;
  }
}

template <typename KV>
hipError_t launch_prefill(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  constexpr int RW = kPrefillRowsPerWave;
  constexpr int NW = kPrefillWaves;
  constexpr int QT = NW * RW;
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  const int nsplit_max = a.partition_blocks > 0 ? a.max_partitions : 1;
  // one dimension, as prefill_item decodes it: whole rounds of quads over the
  // XCDs, each quad's (query tile, key run) members times its 4 heads
  const int64_t members = (int64_t)(a.max_query_len + QT - 1) / QT * nsplit_max;
  const int64_t quads = (int64_t)a.num_seqs * ((a.num_heads + kEngines - 1) / kEngines);
  const int64_t nwg = kXcds * ((quads + kXcds - 1) / kXcds) * members * kEngines;
  if (nwg > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  if constexpr (std::is_same<KV, bf16_t>::value) {
    // With one query tile per sequence and one query head per kv head, each
    // workgroup stages K/V that no other workgroup of the launch reads (unless
    // sequences share prefix blocks): they are streamed past the caches, as
    // decode streams its K/V (long prefixes split over the keys: 304 -> 281 us).
    // Otherwise the query tiles and the heads of a kv head re-read them from
    // the L2, where the hint would evict them early (prefix-cache prefill, 256
    // query rows over a shared prefix: 413 -> 478 us with it).
    const bool stream_kv = members == nsplit_max && a.group == 1;
    if (head_dim == 64) {
      if (stream_kv)
        hipLaunchKernelGGL((prefill_x32_kernel<64, NW, true>), grid, dim3(64 * NW), 0, stream, a);
      else
        hipLaunchKernelGGL((prefill_x32_kernel<64, NW, false>), grid, dim3(64 * NW), 0, stream, a);
    } else {
      if (stream_kv)
        hipLaunchKernelGGL((prefill_x32_kernel<128, NW, true>), grid, dim3(64 * NW), 0, stream, a);
      else
        hipLaunchKernelGGL((prefill_x32_kernel<128, NW, false>), grid, dim3(64 * NW), 0, stream, a);
    }
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((prefill_mfma_kernel<KV, 64, RW, NW>), grid, dim3(64 * NW), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<KV, 128, RW, NW>), grid, dim3(64 * NW), 0, stream, a);
  }
  if (a.partition_blocks > 0 && nsplit_max > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid((a.max_query_len + QT - 1) / QT * kMergeParts, a.num_heads, a.num_seqs);
    if (head_dim == 64)
      hipLaunchKernelGGL((prefill_merge_kernel<64, QT>), mgrid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_merge_kernel<128, QT>), mgrid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  return launch_prefill<bf16_t>(a, head_dim, stream);
}

hipError_t launch_prefill_mfma_fp8(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  return launch_prefill<fp8_t>(a, head_dim, stream);
}

}  // namespace pa
