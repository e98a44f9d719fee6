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
// Butterfly steps on the VALU instead of the LDS crossbar (ds_bpermute).  Each combines the
// values of lanes i and i ^ off; the result of each step has the same bits in both lanes (the
// operations are commutative), as a shuffle-based butterfly would give.
//   off 32, 16: v_permlane32_swap / v_permlane16_swap of a register with itself leave the lower
//     lane's value in the first result and the upper lane's in the second, in both lanes;
//   off < 16:   a DPP row rotation by off.  Rotation by 8 is exactly lane ^ 8 within a 16-lane
//     row; rotation by 4, 2, 1 equals lane ^ off once the values are already equal under
//     lane ^ 2 off, ..., lane ^ 8 (they are, when the steps run from 32 down, as in wave_sum).
__device__ __forceinline__ uint2 swap_halves(float v, int off) {
  const uint32_t u = __float_as_uint(v);
  const auto s = off == 32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return make_uint2(s[0], s[1]);
}
template <int ROR>
__device__ __forceinline__ float row_ror(float v) {
  static_assert(ROR >= 1 && ROR <= 15, "DPP row rotation");
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v),
                                                    0x120 + ROR, 0xf, 0xf, false));
}
// v(lane) + v(lane ^ off) for off in {8, 16, 32}, with no precondition on v.
__device__ __forceinline__ float add_xor(float v, int off) {
  if (off == 8) return v + row_ror<8>(v);
  const uint2 s = swap_halves(v, off);
  return __uint_as_float(s.x) + __uint_as_float(s.y);
}
__device__ __forceinline__ float wave_max(float v) {
  uint2 s = swap_halves(v, 32);
  v = fmaxf(__uint_as_float(s.x), __uint_as_float(s.y));
  s = swap_halves(v, 16);
  v = fmaxf(__uint_as_float(s.x), __uint_as_float(s.y));
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = add_xor(v, 32);
  v = add_xor(v, 16);
  v = add_xor(v, 8);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
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

// ------------------------------------------------------------------ projection on MFMA
// x' = x P for bf16 rows x at fp32 accuracy: every fp32 entry of P is the exact sum of three bf16
// parts (RNE of P, of the remainder, of the remainder's remainder: 8 + 8 + 8 significand bits),
// so every product of a bf16 x with a part is exact and only the fp32 accumulation rounds.
// v_mfma_f32_16x16x32_bf16 lane layout: A lane l holds row l % 16, k = 8 (l / 16) + e (e = 0..7)
// of a 32-wide k-step; B lane l holds column l % 16, the same k; D register r holds row
// 4 (l / 16) + r, column l % 16.  Every bf16 projection in the library (queries before their
// selection, keys before the cache, in every kernel) is this one sequence of operations, so a
// row's x' does not depend on the kernel that computed it.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split3(float p, uint32_t &h, uint32_t &m, uint32_t &l) {
  h = pack_bf16x2(p, 0.0f) & 0xffffu;
  const float r1 = p - bf16_to_f32(static_cast<uint16_t>(h));
  m = pack_bf16x2(r1, 0.0f) & 0xffffu;
  const float r2 = r1 - bf16_to_f32(static_cast<uint16_t>(m));
  l = pack_bf16x2(r2, 0.0f) & 0xffffu;
}

// The three parts of 16 columns of P [D][D] (D = 32 KS) as this lane's B operands.
template <int KS> struct PParts {
  u32x4_t h[KS], m[KS], l[KS];
};

// Columns col0 .. col0 + 15 of P; lane l takes column col0 + l % 16 (at most col_max), rows
// 32 st + 8 (l / 16) + e.  load_p_raw issues the loads, split_p_parts turns the values into the
// three parts (callers that want other loads in flight behind P's issue them in between).
template <int KS>
__device__ __forceinline__ void load_p_raw(const float *__restrict__ P, int col0,
                                           float (&v)[KS][8], int col_max = 32 * KS - 1) {
  constexpr int D = 32 * KS;
  const int lane = threadIdx.x & 63;
  const float *pc = P + (8 * (lane >> 4)) * D + min(col0 + (lane & 15), col_max);
#pragma unroll
  for (int st = 0; st < KS; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[st][e] = pc[(32 * st + e) * D];
}

template <int KS>
__device__ __forceinline__ void split_p_parts(const float (&v)[KS][8], PParts<KS> &pp) {
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    uint32_t h[8], mi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split3(v[st][e], h[e], mi[e], lo[e]);
    pp.h[st] = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
    pp.m[st] = u32x4_t{mi[0] | mi[1] << 16, mi[2] | mi[3] << 16, mi[4] | mi[5] << 16,
                       mi[6] | mi[7] << 16};
    pp.l[st] = u32x4_t{lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16,
                       lo[6] | lo[7] << 16};
  }
}

template <int KS>
__device__ __forceinline__ void load_p_parts(const float *__restrict__ P, int col0,
                                             PParts<KS> &pp) {
  float v[KS][8];
  load_p_raw<KS>(P, col0, v);
  split_p_parts<KS>(v, pp);
}

// This lane's A operand of one bf16 row x [32 KS]: x[32 st + 8 (lane / 16) .. + 7], st = 0..KS-1.
template <int KS>
__device__ __forceinline__ void load_a_row(const uint16_t *row, u32x4_t (&a)[KS]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int st = 0; st < KS; ++st)
    a[st] = *reinterpret_cast<const u32x4_t *>(row + 32 * st + 8 * (lane >> 4));
}

// A 16 x 16 tile of x' = x P: 16 rows (A) by the 16 columns whose parts are pp.
template <int KS>
__device__ __forceinline__ f32x4_t proj_mfma(const u32x4_t (&a)[KS], const PParts<KS> &pp) {
  f32x4_t acc_h = {0.0f, 0.0f, 0.0f, 0.0f}, acc_l = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a[st]);
    acc_l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, pp.l[st]),
                                                    acc_l, 0, 0, 0);
    acc_l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, pp.m[st]),
                                                    acc_l, 0, 0, 0);
    acc_h = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, pp.h[st]),
                                                    acc_h, 0, 0, 0);
  }
  f32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = acc_h[i] + acc_l[i];
  return r;
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

// The scan in parts, for callers that keep the slots' loads in flight behind other work:
// h2o_victim_load requests one batch (thread tid's slots s0 + 256 i, s0 = base + tid),
// h2o_victim_fold ranks it into the thread's (key, slot), h2o_victim_reduce takes the workgroup's
// minimum.  One batch covers 256 * kVictimBatch slots.
constexpr int kVictimBatch = 16;  // slots per thread whose loads are in flight together

struct H2OVictimBatch {
  float mv[kVictimBatch];
  int pv[kVictimBatch];
};

__device__ __forceinline__ void h2o_victim_load(const float *mass, const int32_t *pos,
                                                int n_slots, int s0, H2OVictimBatch &bt) {
#pragma unroll
  for (int i = 0; i < kVictimBatch; ++i) {  // unconditional loads (clamped), validity in the fold
    const int s = min(s0 + 256 * i, n_slots - 1);
    bt.pv[i] = pos[s];
    bt.mv[i] = mass[s];
  }
}

__device__ __forceinline__ void h2o_victim_fold(const H2OVictimBatch &bt, int n_slots, int s0,
                                                int limit, uint64_t &key, int &slot) {
#pragma unroll
  for (int i = 0; i < kVictimBatch; ++i) {
    const int pv = s0 + 256 * i < n_slots ? bt.pv[i] : -1;
    if (pv >= 0 && pv <= limit)
      h2o_keep_min(key, slot,
                   (static_cast<uint64_t>(__float_as_uint(bt.mv[i])) << 32) |
                       static_cast<uint32_t>(0x7fffffff - pv),
                   s0 + 256 * i);
  }
}

__device__ __forceinline__ int h2o_victim_reduce(uint64_t key, int slot) {
  __shared__ uint64_t s_key[4];
  __shared__ int s_slot[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

__device__ __forceinline__ int h2o_pick_victim(const float *mass, const int32_t *pos, int n_slots,
                                               int limit) {
  uint64_t key = ~0ull;
  int slot = 0x7fffffff;
  for (int s0 = threadIdx.x; s0 < n_slots; s0 += 256 * kVictimBatch) {
    H2OVictimBatch bt;
    h2o_victim_load(mass, pos, n_slots, s0, bt);
    __builtin_amdgcn_sched_barrier(0);
    h2o_victim_fold(bt, n_slots, s0, limit, key, slot);
  }
  return h2o_victim_reduce(key, slot);
}

// ------------------------------------------------------------------ launch parameter blocks
struct DecodeArgs {
  const void *kp;        // [B][Hkv][d_store][T_cap]
  const void *v;         // [B][Hkv][T_cap][d]
  const float *q_proj;   // [B][Hq][d]
  const uint32_t *mask;  // [B][Hq][d/32]
  float *mass;           // [B][Hkv][T_cap] or nullptr
  float *out;            // [B][Hq][d]
  // Arrival counters of the cross-workgroup merge, each tagged with the call's epoch in its high
  // 32 bits (arrive_last): a word left by another call, or garbage, is never taken
  // for this call's count, so the workspace needs no clearing.
  uint64_t *counters;      // [B*Hkv]
  uint64_t *run_counters;  // [B*Hkv][run_stride]: per run of splits (two-level merge)
  int run_stride;
  uint32_t epoch;        // nonzero, one more than the previous call's (mod 2^32, 0 skipped)
  float *partials;       // [B][Hq][S][d+2]  (m, l, o[d]) in log2 units
  float *scores;         // [B][Hq][T_cap]   log2-domain scores (mass mode only)
  int B, Hq, Hkv, d, d_store, T_cap, len;
  int S;                 // splits per (b, g)
  int tail_last;         // split-T grid order: 1 deals every group's last split after all the
                         // others (see decode_kernel), 0 the (split, KV head, batch) order
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

// Compute units of the current device (read once per device, then cached).
int device_cu_count();
// A fresh nonzero epoch for a call's arrival counters (process-wide sequence).
uint32_t next_epoch();

// Launch geometry of the split-T decode kernel for a storage dtype (0 f32, 1 bf16), group size
// G, groups = B * Hkv (0: the finest layout, the most splits), context length len and the
// device's compute units.
DecodeLayout decode_layout(int dtype, int G, int groups, int len, int cus);
// aqua_decode takes the short-context kernel (workgroups of 256 tokens that split the union of
// K' rows over their wavefronts) up to this many tokens, the split-T kernel above it.
constexpr int kDecodeShortMax = 4096;
constexpr int kShortChunk = 256;  // tokens per workgroup of the short-context kernel
constexpr int kMergeFan = 8;      // splits per run of the two-level merge
// forms of the short-context kernel: aqua_decode, aqua_decode_step, aqua_h2o_step
enum ShortMode { kShortPlain = 0, kShortStep = 1, kShortH2O = 2 };
bool decode_short(int len, int groups, int cus);  // the short kernel serves this decode
// partials per head that aqua_decode writes (groups = B * Hkv)
int decode_splits(int dtype, int G, int groups, int len, int cus);
size_t decode_workspace_bytes(int dtype, int B, int Hq, int Hkv, int d, int T_cap);
void decode_workspace_carve(void *ws, int dtype, int B, int Hq, int Hkv, int d, int T_cap,
                            DecodeArgs &a);

hipError_t launch_select(const void *q, int qdt, int N, int d, const float *P, int d_sel, int k,
                         float *q_proj, uint32_t *mask, int16_t *idx, hipStream_t s);
hipError_t launch_project_keys(int dtype, const void *k_raw, const void *v_raw, const float *P,
                               int B, int Hkv, int n, int d, int d_store, int T_cap, int len0,
                               const int32_t *slots, void *kp, void *v, hipStream_t s);
hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s);
// the split-T kernel (per storage dtype, plain or fused) and the short-context kernel (mode:
// 0 plain, 1 fused decode step, 2 fused H2O step), each in its own translation unit
hipError_t launch_split_bf16(const DecodeArgs &a, const DecodeLayout &L, hipStream_t s);
hipError_t launch_split_step_bf16(const DecodeArgs &a, const DecodeLayout &L, hipStream_t s);
hipError_t launch_split_f32(const DecodeArgs &a, const DecodeLayout &L, bool fused,
                            hipStream_t s);
hipError_t launch_short_bf16(const DecodeArgs &a, const H2OArgs &h, int mode, hipStream_t s);
hipError_t launch_short_f32(const DecodeArgs &a, const H2OArgs &h, int mode, hipStream_t s);
hipError_t launch_decode_step(int dtype, const DecodeArgs &a, hipStream_t s);
hipError_t launch_h2o_step(int dtype, const DecodeArgs &a, const H2OArgs &h, hipStream_t s);
size_t prefill_workspace_bytes(int B, int Hq, int Lq);
hipError_t launch_prefill(const void *kp, const void *v, int B, int Hq, int Hkv, int d_store,
                          int T_cap, const void *q, int Lq, int pos0, const float *P, int d_sel,
                          int k, float scale, float *out, float *q_proj_out, uint32_t *mask_out,
                          void *ws, hipStream_t s);
hipError_t launch_h2o_victim(float *mass, int32_t *slot_pos, int B, int Hkv, int n_slots,
                             int t_new, int recent, int32_t *victim, hipStream_t s);
size_t gram_workspace_bytes(int64_t n, int d);
hipError_t launch_gram(int dtype, const void *x, int64_t n, int d, double *g, void *ws,
                       hipStream_t s);
hipError_t launch_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink,
                              hipStream_t s);
hipError_t launch_h2o_init(int dtype, const void *kp_full, const void *v_full,
                           const float *mass_full, int B, int Hkv, int d, int d_store,
                           int T_cap_full, int len, int heavy, int recent, void *kp, void *v,
                           float *mass, int32_t *slot_pos, hipStream_t s);

}  // namespace aqua
