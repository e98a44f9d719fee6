// H2O eviction for a compact per-(b, g) cache (AQUA combined with H2O token eviction: abstract of
// arXiv 2509.11155; edgentiq blog, "Key Advantages").  Every token attended at a step gains
// probability mass, a token outside the cache never does, and floating-point addition of
// non-negative terms never decreases a sum, so a token once ranked below every cached heavy
// hitter stays below them.  Each step therefore evicts exactly one slot: the non-recent slot
// ranked lowest by (mass descending, position ascending).
//
// Eviction: one workgroup per (b, g) picks the victim with h2o_pick_victim (the rule the fused H2O step
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

// ------------------------------------------------------------------ starting state
// The compact cache at the start of H2O decoding: for each (b, g), the `heavy` positions ranked
// highest by (mass descending, position ascending) among the positions older than the recent
// window, [0, n_old) with n_old = len - recent, in ascending position order in slots
// 0 .. heavy-1, then the recent positions [n_old, len) in slots heavy .. heavy+recent-1.
//
// Selection, one 1024-thread workgroup per (b, g): the key of position p is
// (mass bits << 32) | (0x7fffffff - p), so a larger key ranks higher and no two keys are equal
// (masses are >= +0, so their bits order like their values).  The heavy-th largest key T is built
// MSB first: bit b of T is kept iff at least `heavy` keys are >= T | bit b, and the search stops
// as soon as exactly `heavy` keys are >= T (it always ends with exactly `heavy`: the keys are
// distinct).  The positions with key >= T are then written in ascending order, each thread
// compacting a contiguous range of positions at its offset from a workgroup prefix sum.
constexpr int kInitThreads = 1024;

__device__ __forceinline__ uint64_t h2o_rank_key(const float *m, int p) {
  return (static_cast<uint64_t>(__float_as_uint(m[p])) << 32) |
         static_cast<uint32_t>(0x7fffffff - p);
}

__global__ __launch_bounds__(kInitThreads) void h2o_init_select_kernel(
    const float *__restrict__ mass_full, int T_cap_full, int n_old, int heavy, int recent,
    int32_t *__restrict__ slot_pos, int n_slots) {
  constexpr int NWAVE = kInitThreads / 64;
  __shared__ int s_cnt[NWAVE];
  const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float *m = mass_full + static_cast<size_t>(bg) * T_cap_full;
  int32_t *sp = slot_pos + static_cast<size_t>(bg) * n_slots;

  // workgroup sum of one int per thread (every thread gets it)
  auto block_sum = [&](int n) -> int {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
    if (lane == 0) s_cnt[w] = n;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) tot += s_cnt[x];
    __syncthreads();  // s_cnt is rewritten by the next call
    return tot;
  };

  uint64_t T = 0;
  if (heavy > 0) {
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t c = T | (1ull << bit);
      int n = 0;
      for (int p = tid; p < n_old; p += kInitThreads) n += h2o_rank_key(m, p) >= c ? 1 : 0;
      const int cnt = block_sum(n);  // uniform
      if (cnt >= heavy) {
        T = c;
        if (cnt == heavy) break;
      }
    }
    // ascending compaction of the positions with key >= T
    const int chunk = (n_old + kInitThreads - 1) / kInitThreads;
    const int p0 = min(tid * chunk, n_old), p1 = min(p0 + chunk, n_old);
    int mine = 0;
    for (int p = p0; p < p1; ++p) mine += h2o_rank_key(m, p) >= T ? 1 : 0;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_cnt[w] = incl;
    __syncthreads();
    int at = incl - mine;
    for (int x = 0; x < w; ++x) at += s_cnt[x];
    for (int p = p0; p < p1; ++p)
      if (h2o_rank_key(m, p) >= T) sp[at++] = p;
  }
  for (int i = tid; i < recent; i += kInitThreads) sp[heavy + i] = n_old + i;
}

// Gathers each slot's K' column, V row and mass from the full cache (64 slots per workgroup).
template <typename KT>
__global__ __launch_bounds__(256) void h2o_init_gather_kernel(
    const KT *__restrict__ kp_full, const KT *__restrict__ v_full,
    const float *__restrict__ mass_full, int T_cap_full, int d, int d_store,
    const int32_t *__restrict__ slot_pos, int n_slots, KT *__restrict__ kp, KT *__restrict__ v,
    float *__restrict__ mass) {
  __shared__ int s_pos[64];
  const int bg = blockIdx.y, s0 = blockIdx.x * 64, tid = threadIdx.x;
  const int ns = min(64, n_slots - s0);
  if (tid < ns) s_pos[tid] = slot_pos[static_cast<size_t>(bg) * n_slots + s0 + tid];
  __syncthreads();
  const size_t full0 = static_cast<size_t>(bg) * T_cap_full;
  const size_t cmp0 = static_cast<size_t>(bg) * n_slots;
  for (int e = tid; e < d_store * 64; e += 256) {
    const int i = e >> 6, s = e & 63;
    if (s < ns)
      kp[(static_cast<size_t>(bg) * d_store + i) * n_slots + s0 + s] =
          kp_full[(static_cast<size_t>(bg) * d_store + i) * T_cap_full + s_pos[s]];
  }
  const int vec = d * static_cast<int>(sizeof(KT)) / 16;  // 16-byte pieces per V row
  for (int e = tid; e < ns * vec; e += 256) {
    const int s = e / vec, c = e - s * vec;
    reinterpret_cast<uint4 *>(v + (cmp0 + s0 + s) * d)[c] =
        reinterpret_cast<const uint4 *>(v_full + (full0 + s_pos[s]) * d)[c];
  }
  if (tid < ns) mass[cmp0 + s0 + tid] = mass_full[full0 + s_pos[tid]];
}

}  // namespace

hipError_t launch_h2o_init(int dtype, const void *kp_full, const void *v_full,
                           const float *mass_full, int B, int Hkv, int d, int d_store,
                           int T_cap_full, int len, int heavy, int recent, void *kp, void *v,
                           float *mass, int32_t *slot_pos, hipStream_t s) {
  const int n_slots = heavy + recent;
  h2o_init_select_kernel<<<dim3(B * Hkv), dim3(kInitThreads), 0, s>>>(
      mass_full, T_cap_full, len - recent, heavy, recent, slot_pos, n_slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((n_slots + 63) / 64, B * Hkv);
  if (dtype == 1)
    h2o_init_gather_kernel<bf16_t><<<grid, dim3(256), 0, s>>>(
        static_cast<const bf16_t *>(kp_full), static_cast<const bf16_t *>(v_full), mass_full,
        T_cap_full, d, d_store, slot_pos, n_slots, static_cast<bf16_t *>(kp),
        static_cast<bf16_t *>(v), mass);
  else
    h2o_init_gather_kernel<float><<<grid, dim3(256), 0, s>>>(
        static_cast<const float *>(kp_full), static_cast<const float *>(v_full), mass_full,
        T_cap_full, d, d_store, slot_pos, n_slots, static_cast<float *>(kp),
        static_cast<float *>(v), mass);
  return hipGetLastError();
}

hipError_t launch_h2o_victim(float *mass, int32_t *slot_pos, int B, int Hkv, int n_slots,
                             int t_new, int recent, int32_t *victim, hipStream_t s) {
  h2o_victim_kernel<<<dim3(B * Hkv), dim3(256), 0, s>>>(mass, slot_pos, n_slots, t_new, recent,
                                                        victim);
  return hipGetLastError();
}

}  // namespace aqua
