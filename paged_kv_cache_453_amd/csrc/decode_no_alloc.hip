// pa_decode_no_alloc: pa_decode followed by pa_decode_splitk_reduce, with the
// split-K partials kept in a fixed device buffer that the library owns, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The buffer is a file-scope __device__ array, one copy per GPU the library
// runs on, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in symbol): the first call
// on a device looks up that device's copy with hipGetSymbolAddress, with the
// device current, and every launch takes that address.  Every call on a GPU
// uses the same copy, so calls that overlap on one GPU (two streams, two
// threads) race on it; calls on one stream are ordered and safe.  Nothing in
// it has to start at zero: each split sequence's partitions are written by the
// decode before the merge reads them, and nothing else is read.
#include <mutex>

#include "pa.h"
#include "pa_launch.h"

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up once per device, then cached).
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_no_alloc_scratch_bytes(void) { return kScratchBytes; }

int pa_decode_no_alloc(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                       int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int64_t num_blocks,
                       int max_context_len, float scale, int partition_size, pa_dtype dtype,
                       hipStream_t stream) {
  // the checks pa_decode makes, before any HIP call
  const int chk = pa::check_decode_args(out, query, key_cache, value_cache, block_tables,
                                        context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                        block_size, max_blocks_per_seq, num_blocks,
                                        max_context_len, partition_size, dtype);
  if (chk != PA_OK) return chk;
  void* ws = nullptr;
  if (partition_size > 0 && num_seqs > 0) {
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                  partition_size);
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    const int st = scratch_of_current_device(&ws);
    if (st != PA_OK) return st;
  }
  const int st = pa_decode(out, query, key_cache, value_cache, block_tables, context_lens,
                           shared_prefix_blocks, num_seqs, num_heads, num_kv_heads, head_dim,
                           block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                           partition_size, ws, ws ? kScratchBytes : 0, dtype, stream);
  if (st != PA_OK || partition_size <= 0 || num_seqs == 0) return st;
  return pa_decode_splitk_reduce(out, ws, kScratchBytes, context_lens, num_seqs, num_heads,
                                 head_dim, max_context_len, partition_size, dtype, stream);
}

}  // extern "C"
