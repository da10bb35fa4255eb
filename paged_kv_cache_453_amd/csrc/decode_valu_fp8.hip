// Instantiates the vector-ALU decode kernels for FP8 (E4M3) caches with fp32 or
// bf16 queries (head_dim 64 and 128, up to 4 query heads per kv head).
#include "decode_valu.h"

namespace pa {

hipError_t launch_decode_valu_fp8(const DecodeArgs& a, int head_dim, bool bf16_query,
                                  hipStream_t stream) {
  if (bf16_query)
    return head_dim == 64 ? launch_decode_t<bf16_t, fp8_t, 64>(a, stream)
                          : launch_decode_t<bf16_t, fp8_t, 128>(a, stream);
  return head_dim == 64 ? launch_decode_t<float, fp8_t, 64>(a, stream)
                        : launch_decode_t<float, fp8_t, 128>(a, stream);
}

}  // namespace pa
