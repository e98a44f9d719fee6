// Internal declarations shared by the libaqua host layer and its HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aqua {

// ------------------------------------------------------------------ bf16 storage helpers
// bf16 is the upper half of an fp32 bit pattern.  Widening is exact; narrowing rounds to
// nearest with ties to even (v_cvt_pk_bf16_f32: branch-free; identical to adding 0x7fff plus
// the lowest kept bit and truncating, for every finite input).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) {
  return __uint_as_float(pair & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Two fp32 values to a bf16 pair (lo in bits 0-15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Storage element types: float (AQUA_F32) or raw bf16 bits (AQUA_BF16).
using bf16_t = uint16_t;

template <typename T> __device__ __forceinline__ float load_elem(const T *p);
template <> __device__ __forceinline__ float load_elem<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_elem<bf16_t>(const bf16_t *p) {
  return bf16_to_f32(*p);
}
template <typename T> __device__ __forceinline__ T store_elem(float f);
template <> __device__ __forceinline__ float store_elem<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t store_elem<bf16_t>(float f) {
  return f32_to_bf16_rne(f);
}

// ------------------------------------------------------------------ wave helpers (wave64)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Top-k of one row of D = 64 * E values held by a wavefront, lane l holding dims l + 64 e.
// Magnitudes are compared exactly, as the fp32 bit patterns with the sign cleared (+0 and -0
// tie, denormals are not flushed); equal magnitudes go to the lower index.  Exactly k flags are
// set, all at dims < d_sel (callers guarantee 1 <= k <= d_sel <= 64 E).
// Threshold search: the k-th largest key T is built MSB first (keep bit b of T iff at least k
// keys are >= T | bit b), stopping early once exactly k keys are >= the running threshold.
// Keys of dims >= d_sel are -1, below every magnitude.  If the search ends with more than k
// keys >= T (ties at T), the keys > T are kept and the ties are taken in index order.  Per
// bit: two compares and two ballot popcounts, the rest is scalar.
template <int E>
__device__ __forceinline__ void wave_topk_threshold(const float (&x)[E], int d_sel, int k,
                                                    bool (&sel)[E]) {
  const int lane = threadIdx.x & 63;
  int u[E];
#pragma unroll
  for (int e = 0; e < E; ++e)
    u[e] = (lane + 64 * e) < d_sel ? static_cast<int>(__float_as_uint(x[e]) & 0x7fffffffu) : -1;
  int T = 0;
  bool exact = (d_sel == k);
  if (!exact) {
    for (int bit = 30; bit >= 0; --bit) {
      const int c = T | (1 << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(u[e] >= c));
      if (cnt >= k) {
        T = c;
        if (cnt == k) {
          exact = true;
          break;
        }
      }
    }
  }
  if (exact) {
#pragma unroll
    for (int e = 0; e < E; ++e) sel[e] = u[e] >= T;
    return;
  }
  int need = k;
#pragma unroll
  for (int e = 0; e < E; ++e) need -= __popcll(__ballot(u[e] > T));
  int before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(u[e] == T);
    const int rank = before + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                  static_cast<uint32_t>(b >> 32),
                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u)));
    sel[e] = u[e] > T || (u[e] == T && rank < need);
    before += __popcll(b);
  }
}

// A workgroup barrier that orders LDS traffic only: unlike __syncthreads, whose fence waits
// for every outstanding global load too, it lets loads issued earlier stay in flight.  The
// empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ H2O eviction rule
// Among the slots of one (b, g) holding a position <= limit (t_new - recent), the one ranked lowest
// by (mass descending, position ascending): the minimum of the 64-bit key (mass bits,
// 0x7fffffff - position), mass >= 0 so that its fp32 bits order like the value; equal keys go
// to the lower slot.  Called by every thread of a 256-thread workgroup (it holds barriers);
// returns the slot, or -1 if no slot qualifies, in every thread.
__device__ __forceinline__ void h2o_keep_min(uint64_t &key, int &slot, uint64_t k2, int s2) {
  if (k2 < key || (k2 == key && s2 < slot)) {
    key = k2;
    slot = s2;
  }
}

__device__ __forceinline__ int h2o_pick_victim(const float *mass, const int32_t *pos, int n_slots,
                                               int limit) {
  __shared__ uint64_t s_key[4];
  __shared__ int s_slot[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint64_t key = ~0ull;
  int slot = 0x7fffffff;
  constexpr int BATCH = 16;  // slots per thread whose loads are in flight together
  for (int s0 = tid; s0 < n_slots; s0 += 256 * BATCH) {
    float mv[BATCH];
    int pv[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {  // unconditional loads (clamped), validity applied below
      const int s = min(s0 + 256 * i, n_slots - 1);
      pv[i] = pos[s];
      mv[i] = mass[s];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (s0 + 256 * i >= n_slots) pv[i] = -1;
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (pv[i] >= 0 && pv[i] <= limit)
        h2o_keep_min(key, slot,
                     (static_cast<uint64_t>(__float_as_uint(mv[i])) << 32) |
                         static_cast<uint32_t>(0x7fffffff - pv[i]),
                     s0 + 256 * i);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t k2 = __shfl_xor(key, off, 64);
    const int s2 = __shfl_xor(slot, off, 64);
    h2o_keep_min(key, slot, k2, s2);
  }
  if (lane == 0) {
    s_key[w] = key;
    s_slot[w] = slot;
  }
  __syncthreads();
  key = s_key[0];
  slot = s_slot[0];
  for (int x = 1; x < 4; ++x) h2o_keep_min(key, slot, s_key[x], s_slot[x]);
  return key == ~0ull ? -1 : slot;
}

// ------------------------------------------------------------------ launch parameter blocks
struct DecodeArgs {
  const void *kp;        // [B][Hkv][d_store][T_cap]
  const void *v;         // [B][Hkv][T_cap][d]
  const float *q_proj;   // [B][Hq][d]
  const uint32_t *mask;  // [B][Hq][d/32]
  float *mass;           // [B][Hkv][T_cap] or nullptr
  float *out;            // [B][Hq][d]
  uint32_t *counters;    // [B*Hkv], zero between calls
  uint32_t *run_counters;  // [B*Hkv][run_stride]: per run of splits (two-level merge), zero
  int run_stride;
  float *partials;       // [B][Hq][S][d+2]  (m, l, o[d]) in log2 units
  float *scores;         // [B][Hq][T_cap]   log2-domain scores (mass mode only)
  int B, Hq, Hkv, d, d_store, T_cap, len;
  int S;                 // splits per (b, g)
  float qscale;          // scale * log2(e)
  // fused decode step only: raw queries and the new token, selection parameters
  const void *q_raw;     // [B][Hq][d]
  const void *k_new;     // [B][Hkv][d]
  const void *v_new;     // [B][Hkv][d]
  const float *P;        // [d][d]
  float *q_proj_out;     // [B][Hq][d] or nullptr
  uint32_t *mask_out;    // [B][Hq][d/32] or nullptr
  void *kp_w, *v_w;      // the cache, written at column len - 1
  int d_sel, k;
};

// Fused H2O step only: the compact cache's slot positions, the step's position and window, and
// where the evicted slot is reported.
struct H2OArgs {
  int32_t *slot_pos;  // [B][Hkv][n_slots], n_slots = T_cap = len
  int32_t *victim;    // [B][Hkv]
  int t_new, recent;
};

struct DecodeLayout {
  int waves;        // waves per workgroup
  int tokens_wave;  // tokens per wave
  int split;        // tokens per workgroup (= waves * tokens_wave)
};

// Launch geometry of the split-T decode kernel for a storage dtype (0 f32, 1 bf16), group size
// G, groups = B * Hkv (0: the finest layout, the most splits) and context length len.
DecodeLayout decode_layout(int dtype, int G, int groups, int len);
// aqua_decode takes the short-context kernel (workgroups of 256 tokens that split the union of
// K' rows over their wavefronts) up to this many tokens, the split-T kernel above it.
constexpr int kDecodeShortMax = 4096;
bool decode_short(int len);
// partials per head that aqua_decode writes (groups = B * Hkv)
int decode_splits(int dtype, int G, int groups, int len);
size_t decode_workspace_bytes(int dtype, int B, int Hq, int Hkv, int d, int T_cap);
void decode_workspace_carve(void *ws, int dtype, int B, int Hq, int Hkv, int d, int T_cap,
                            DecodeArgs &a);

hipError_t launch_select(const void *q, int qdt, int N, int d, const float *P, int d_sel, int k,
                         float *q_proj, uint32_t *mask, int16_t *idx, hipStream_t s);
hipError_t launch_project_keys(int dtype, const void *k_raw, const void *v_raw, const float *P,
                               int B, int Hkv, int n, int d, int d_store, int T_cap, int len0,
                               const int32_t *slots, void *kp, void *v, hipStream_t s);
hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_step(int dtype, const DecodeArgs &a, hipStream_t s);
hipError_t launch_h2o_step(int dtype, const DecodeArgs &a, const H2OArgs &h, hipStream_t s);
size_t prefill_workspace_bytes(int B, int Hq, int Lq);
hipError_t launch_prefill(const void *kp, const void *v, int B, int Hq, int Hkv, int d_store,
                          int T_cap, const void *q, int Lq, int pos0, const float *P, int d_sel,
                          int k, float scale, float *out, float *q_proj_out, uint32_t *mask_out,
                          void *ws, hipStream_t s);
hipError_t launch_h2o_victim(float *mass, int32_t *slot_pos, int B, int Hkv, int n_slots,
                             int t_new, int recent, int32_t *victim, hipStream_t s);

}  // namespace aqua
