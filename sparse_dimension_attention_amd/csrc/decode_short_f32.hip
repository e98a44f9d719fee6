// The short-context decode kernel for fp32 storage (all three modes).  Kernel templates:
// decode_kernels.h.
#include "decode_kernels.h"

namespace aqua {

hipError_t launch_short_f32(const DecodeArgs &a, const H2OArgs &h, int mode, hipStream_t s) {
  if (mode == kShortH2O) return launch_short_t<float, kShortH2O>(a, h, s);
  if (mode == kShortStep) return launch_short_t<float, kShortStep>(a, h, s);
  return launch_short_t<float, kShortPlain>(a, h, s);
}

}  // namespace aqua
