// Instantiates the vector-ALU decode kernels for bf16 caches (head_dim 64 and 128).
#include "decode_valu.h"

namespace pa {

hipError_t launch_decode_valu_bf16(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_decode_t<bf16_t, bf16_t, 64>(a, stream)
                        : launch_decode_t<bf16_t, bf16_t, 128>(a, stream);
}

}  // namespace pa
