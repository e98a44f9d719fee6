// The split-T decode kernel for bf16 storage, plain form (aqua_decode past the short-context
// length).  Kernel templates: decode_kernels.h.
#include "decode_kernels.h"

namespace aqua {

hipError_t launch_split_bf16(const DecodeArgs &a, const DecodeLayout &L, hipStream_t s) {
  return launch_split_t<bf16_t, false>(a, L, s);
}

}  // namespace aqua
