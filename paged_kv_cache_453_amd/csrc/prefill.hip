// Causal chunked prefill over a paged KV cache on bf16 matrix cores (MFMA).
//
// Chunked prefill splits one prompt's prefill over several rounds (xdnf.cn
// article, section 六.4); each chunk's queries sit at the last C positions of
// their sequence and must see every earlier token, the paged prefix included.
// Prefill is compute-bound (xdnf.cn article, section 六.5), so this kernel is a
// tiled flash-attention loop on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation, K/V tiles gathered through the block table.
//
// Tiling.  A workgroup (4 waves) owns 64 query rows of one head of one
// sequence; each wave owns 16 rows.  Keys are processed in tiles of 64 tokens
// (4 cache blocks) staged in LDS: K row-major, V transposed so that the p.V
// product can read its operand along the key axis.
//
// Orientation.  Scores are produced transposed, S^T = K Q^T, and the output as
// O^T = V^T P^T.  In a 16x16 MFMA result, lane l holds column l % 16; with this
// orientation column = query row, so the softmax state of a query row (running
// max, running sum, output rescale) lives in the four lanes l % 16 == row, and
// the probabilities come out of the score MFMA already laid out as the B
// operand of the p.V MFMA.  No transpose of P is needed.
//
// The reduction index of an MFMA may be permuted freely as long as both
// operands use the same permutation; the p.V step uses that freedom to pair
// key groups {4g..4g+3} and {16+4g..16+4g+3} in one 8-element operand.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kQRows = 64;     // query rows per workgroup
constexpr int kKeys = 64;      // keys per tile (4 blocks)
constexpr int kPadK = 8;       // bf16 pad per K row in LDS
constexpr int kPadV = 8;       // bf16 pad per transposed V row in LDS

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;    // k-steps of the score MFMA
  constexpr int DT = D / 16;    // 16-wide output dim tiles
  constexpr int CH = D / 8;     // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) bf16_t sK[kKeys][D + kPadK];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[D][kKeys + kPadV];
  __shared__ int sh_bad;

  const int qtile = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_uniform(tid >> 6);
  const int row = lane & 15;
  const int grp = lane >> 4;
  const int hq = a.num_heads;
  const int kvh = h / a.group;

  const int q0 = a.query_start_loc[s];
  const int q1 = a.query_start_loc[s + 1];
  // rows outside [0, num_query_tokens) cannot be written at all
  if (q0 < 0 || q1 < q0 || q1 > a.num_items) return;
  const int chunk = q1 - q0;
  const int len = a.context_lens[s];
  const int qr0 = qtile * kQRows;
  if (qr0 >= chunk) return;
  const bool bad = chunk > len || chunk > a.max_query_len || len > a.max_blocks_per_seq * kBlock;
  const int prefix = len - chunk;
  const int qi = qr0 + w * 16 + row;           // query row inside the chunk
  const bool qvalid = qi < chunk;
  const int qpos = prefix + qi;                // absolute position of the query
  bf16_t* out = static_cast<bf16_t*>(a.out);

  if (bad) {
    // the whole chunk of this sequence is reported as NaN
    for (int i = tid; i < kQRows * D; i += 256) {
      const int rr = qr0 + i / D;
      if (rr < chunk) out[((int64_t)(q0 + rr) * hq + h) * D + i % D] = 0x7FC0;
    }
    return;
  }
  if (tid == 0) sh_bad = 0;

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[row][32ks + 8grp .. +8].
  bf16x8 qb[KS];
  const bf16_t* qsrc = static_cast<const bf16_t*>(a.query) + ((int64_t)(q0 + qi) * hq + h) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qvalid) {
      qb[ks] = *reinterpret_cast<const bf16x8*>(qsrc + 32 * ks + 8 * grp);
    } else {
      qb[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int qlast = min(chunk, qr0 + kQRows) - 1;
  const int kend = prefix + qlast + 1;         // keys [0, kend) matter to this workgroup
  const int ntiles = (kend + kKeys - 1) / kKeys;
  const float sl2 = a.scale_log2;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const bf16_t* kpool = static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vpool = static_cast<const bf16_t*>(a.v_cache);

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();   // the previous tile has been consumed
    // ---- stage K (row-major) and V (transposed) of keys [64kt, 64kt+64) ----
    for (int ci = tid; ci < kKeys * CH; ci += 256) {
      const int key = ci / CH;
      const int cc = ci - key * CH;
      const int tok = kt * kKeys + key;
      u32x4 kv = u32x4{0u, 0u, 0u, 0u};
      u32x4 vv = u32x4{0u, 0u, 0u, 0u};
      if (tok < kend) {
        const int bid = table[tok / kBlock];
        if (bid >= 0 && (int64_t)bid < a.num_blocks) {
          const int64_t off = (((int64_t)bid * a.num_kv_heads + kvh) * kBlock + tok % kBlock) * D + cc * 8;
          kv = *reinterpret_cast<const u32x4*>(kpool + off);
          vv = *reinterpret_cast<const u32x4*>(vpool + off);
        } else {
          sh_bad = 1;
        }
      }
      *reinterpret_cast<u32x4*>(&sK[key][cc * 8]) = kv;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sVt[cc * 8 + 2 * x][key] = (bf16_t)(vv[x] & 0xffffu);
        sVt[cc * 8 + 2 * x + 1][key] = (bf16_t)(vv[x] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: four 16-key groups ----
    f32x4 sc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sK[16 * nt + row][32 * ks + 8 * grp]);
        sc[nt] = mfma_16x16x32(ka, qb[ks], sc[nt]);
      }
    }
    // lane holds S[query row][key 64kt + 16nt + 4grp + i]
    float tmax = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt * kKeys + 16 * nt + 4 * grp + i;
        const float v = key <= qpos ? sc[nt][i] * sl2 : -INFINITY;
        sc[nt][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m - mn);
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    // probabilities, rounded to bf16 for the p.V MFMA; the running sum adds the
    // rounded values so numerator and denominator use the same weights
    uint32_t pk[4][2];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = (sc[nt][i] == -INFINITY) ? 0.f : exp2f(sc[nt][i] - mn);
        const float p1 = (sc[nt][i + 1] == -INFINITY) ? 0.f : exp2f(sc[nt][i + 1] - mn);
        const uint32_t wpk = pack_bf16x2(p0, p1);
        pk[nt][i / 2] = wpk;
        lsum += bf16_lo(wpk) + bf16_hi(wpk);
      }
    m = mn;

    // ---- O^T += V^T P^T, 32 keys per MFMA ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 pw = u32x4{pk[2 * kk][0], pk[2 * kk][1], pk[2 * kk + 1][0], pk[2 * kk + 1][1]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16_t* vr = &sVt[16 * dt + row][32 * kk + 4 * grp];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[dt] = mfma_16x16x32(va, pb, o[dt]);
      }
    }
  }

  // ---- normalise and store: lane holds O[row][16dt + 4grp + i] ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  __syncthreads();
  const bool poisoned = sh_bad != 0;
  if (qvalid) {
    const float inv = 1.f / lsum;
    bf16_t* dst = out + ((int64_t)(q0 + qi) * hq + h) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2 pk;
      if (poisoned) {
        pk = u32x2{0x7FC07FC0u, 0x7FC07FC0u};
      } else {
        pk[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
        pk[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      }
      *reinterpret_cast<u32x2*>(dst + 16 * dt) = pk;
    }
  }
}

hipError_t launch_prefill_mfma(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  dim3 grid((a.max_query_len + kQRows - 1) / kQRows, a.num_heads, a.num_seqs);
  if (head_dim == 64)
    hipLaunchKernelGGL((prefill_mfma_kernel<64>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<128>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
