// The short-context decode kernel for bf16 storage: aqua_decode and aqua_decode_step up to the
// short-context length, and aqua_h2o_step.  Kernel templates: decode_kernels.h.
#include "decode_kernels.h"

namespace aqua {

hipError_t launch_short_bf16(const DecodeArgs &a, const H2OArgs &h, int mode, hipStream_t s) {
  if (mode == kShortH2O) return launch_short_t<bf16_t, kShortH2O>(a, h, s);
  if (mode == kShortStep) return launch_short_t<bf16_t, kShortStep>(a, h, s);
  return launch_short_t<bf16_t, kShortPlain>(a, h, s);
}

}  // namespace aqua
