// H2O eviction for a compact per-(b, g) cache (AQUA combined with H2O token eviction: abstract of
// arXiv 2509.11155; edgentiq blog, "Key Advantages").  Every token attended at a step gains
// probability mass, a token outside the cache never does, and floating-point addition of
// non-negative terms never decreases a sum, so a token once ranked below every cached heavy
// hitter stays below them.  Each step therefore evicts exactly one slot: the non-recent slot
// ranked lowest by (mass descending, position ascending).
//
// One workgroup per (b, g).  Each slot's rank key is (mass bits, 0x7fffffff - pos) compared as
// a 64-bit unsigned integer (mass >= 0, so its fp32 bit pattern orders like the value); the
// minimum key is the victim.  Reduction: per lane, wave (shuffles), then across wavefronts.
#include "aqua_internal.h"

namespace aqua {
namespace {

__device__ __forceinline__ void keep_min(uint64_t &key, int &slot, uint64_t k2, int s2) {
  if (k2 < key || (k2 == key && s2 < slot)) {
    key = k2;
    slot = s2;
  }
}

__global__ __launch_bounds__(256) void h2o_victim_kernel(float *__restrict__ mass,
                                                         int32_t *__restrict__ slot_pos,
                                                         int n_slots, int t_new, int recent,
                                                         int32_t *__restrict__ victim) {
  __shared__ uint64_t s_key[4];
  __shared__ int s_slot[4];
  const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float *m = mass + static_cast<size_t>(bg) * n_slots;
  int32_t *pos = slot_pos + static_cast<size_t>(bg) * n_slots;
  const int limit = t_new - recent;  // non-recent: position <= limit

  uint64_t key = ~0ull;
  int slot = 0x7fffffff;
  for (int s = tid; s < n_slots; s += 256) {
    const int p = pos[s];
    if (p >= 0 && p <= limit) {
      const uint64_t k2 = (static_cast<uint64_t>(__float_as_uint(m[s])) << 32) |
                          static_cast<uint32_t>(0x7fffffff - p);
      keep_min(key, slot, k2, s);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t k2 = __shfl_xor(key, off, 64);
    const int s2 = __shfl_xor(slot, off, 64);
    keep_min(key, slot, k2, s2);
  }
  if (lane == 0) {
    s_key[w] = key;
    s_slot[w] = slot;
  }
  __syncthreads();
  if (tid == 0) {
    for (int x = 1; x < 4; ++x) keep_min(key, slot, s_key[x], s_slot[x]);
    if (key == ~0ull) {
      victim[bg] = -1;
    } else {
      victim[bg] = slot;
      pos[slot] = t_new;
      m[slot] = 0.0f;
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
