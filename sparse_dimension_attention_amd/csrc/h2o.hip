// H2O eviction for a compact per-(b, g) cache (AQUA combined with H2O token eviction: abstract of
// arXiv 2509.11155; edgentiq blog, "Key Advantages").  Every token attended at a step gains
// probability mass, a token outside the cache never does, and floating-point addition of
// non-negative terms never decreases a sum, so a token once ranked below every cached heavy
// hitter stays below them.  Each step therefore evicts exactly one slot: the non-recent slot
// ranked lowest by (mass descending, position ascending).
//
// One workgroup per (b, g) picks the victim with h2o_pick_victim (the rule the fused H2O step
// applies too): the minimum of the key (mass bits, 0x7fffffff - pos), reduced per lane, per
// wavefront (shuffles), then across wavefronts.
#include "aqua_internal.h"

namespace aqua {
namespace {

__global__ __launch_bounds__(256) void h2o_victim_kernel(float *__restrict__ mass,
                                                         int32_t *__restrict__ slot_pos,
                                                         int n_slots, int t_new, int recent,
                                                         int32_t *__restrict__ victim) {
  const int bg = blockIdx.x;
  float *m = mass + static_cast<size_t>(bg) * n_slots;
  int32_t *pos = slot_pos + static_cast<size_t>(bg) * n_slots;
  const int v = h2o_pick_victim(m, pos, n_slots, t_new - recent);
  if (threadIdx.x == 0) {
    victim[bg] = v;
    if (v >= 0) {
      pos[v] = t_new;
      m[v] = 0.0f;
    }
  }
}

}  // namespace

hipError_t launch_h2o_victim(float *mass, int32_t *slot_pos, int B, int Hkv, int n_slots,
                             int t_new, int recent, int32_t *victim, hipStream_t s) {
  h2o_victim_kernel<<<dim3(B * Hkv), dim3(256), 0, s>>>(mass, slot_pos, n_slots, t_new, recent,
                                                        victim);
  return hipGetLastError();
}

}  // namespace aqua
