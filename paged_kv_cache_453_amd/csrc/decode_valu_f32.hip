// Instantiates the vector-ALU decode kernels for fp32 caches (head_dim 64 and 128).
#include "decode_valu.h"

namespace pa {

hipError_t launch_decode_valu_f32(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_decode_t<float, float, 64>(a, stream)
                        : launch_decode_t<float, float, 128>(a, stream);
}

}  // namespace pa
