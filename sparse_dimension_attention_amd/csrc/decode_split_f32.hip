// The split-T decode kernel for fp32 storage, plain and fused forms.  Kernel templates:
// decode_kernels.h.
#include "decode_kernels.h"

namespace aqua {

hipError_t launch_split_f32(const DecodeArgs &a, const DecodeLayout &L, bool fused,
                            hipStream_t s) {
  return fused ? launch_split_t<float, true>(a, L, s) : launch_split_t<float, false>(a, L, s);
}

}  // namespace aqua
