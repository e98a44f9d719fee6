// Kernel templates of GQA decode attention over each query's selected projected dimensions (AQUA: attention
// computed on the dims kept by projected-query magnitude; digest of arXiv 2509.11155, section
// 方法详解 / 技术框架; edgentiq blog, "How AQUA Works", step 2), split over the context with a
// final flash-decoding style combination of (max, sum, weighted V) partials.
//
// Memory-bound design for one (b, KV group g) and one split of the context per workgroup:
//  * The G query heads of a KV group each keep their own dims; the workgroup reads the K' rows
//    of the union U of those masks, once, and every head uses its own masked q' (zero on dims it
//    did not keep).  K' is dimension-major, so each selected row is a contiguous run of tokens:
//    lane l reads 16 bytes (8 bf16 / 4 fp32 tokens) of a row, a wavefront 1 KiB, fully coalesced,
//    non-temporal; rows outside U are never touched.  Loads are issued a batch ahead of the
//    arithmetic (ping-pong registers), and each workgroup starts its walk over U at its own
//    offset so that concurrent workgroups spread over the HBM channels.
//  * Each wavefront owns a contiguous run of 64 * 16/sizeof(elem) tokens and computes all of
//    its scores before any exponential, so there is no running rescale inside a wavefront.
//    Scores live in log2 units (q' pre-multiplied by scale * log2 e) and use v_exp_f32.
//  * The softmax numerators go through LDS to the V pass, where 16 bytes per lane cover a V
//    row (d = 128 bf16: 16 lanes per token, 4 tokens per wavefront load).
//  * The workgroup's wavefronts merge their (m, l, o) in LDS; the workgroup writes one partial
//    per query head.  The last workgroup of a (b, g) to finish (atomic counter in the
//    workspace) merges all partials of the group, writes the output and resets its counter;
//    past 16 splits per group the merge takes two levels (finish_split).
//  * H2O mass mode additionally stores the raw scores and lets that last workgroup add every
//    token's normalised probability, summed over the group's heads, to its mass.
//
// The fused decode step (FUSED) does a whole step in this one launch: each workgroup projects its
// group's raw queries and the new key (bf16 storage: on MFMA with P's three bf16 parts in
// registers; fp32 storage: on the VALU with P staged in LDS), selects every head's top-k dims
// with wave_topk_threshold, appends the new token's K' and V to the cache (the workgroup that
// holds the new position), and attends over the cached tokens plus the new one, taken from LDS.
// Up to the short-context length the fused step runs on the short kernel instead (256-token
// workgroups, the same prologue), as the fused H2O step does.
#pragma once

#include <type_traits>

#include "aqua_internal.h"

namespace aqua {
namespace {

constexpr int kUnroll = 8;

template <typename KT> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void unpack(const uint4 &r, float (&f)[8]) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void unpack(const uint4 &r, float (&f)[4]) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const void *p) {
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}
// Cross-workgroup hand-off without cache-wide fences.  Partials and scores are written and read
// with system-scope relaxed atomics (sc0 sc1: written through / read past every non-coherent
// cache level); the writer drains its stores (s_waitcnt) before the workgroup barrier that
// precedes the counter increment, and the reader issues its loads only after the counter RMW
// has told it that it is last.  An agent-scope fence here would instead write back and
// invalidate the whole L2 of the XCD once per workgroup, which stalls every streaming load.
__device__ __forceinline__ void publish(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Counts this workgroup's arrival at a counter shared by `total` workgroups of one call; true in
// the last to arrive.  The word holds (epoch << 32) | count.  An arrival first lifts the word to
// (epoch, 0) with an atomic max (no return; a word already at this epoch keeps its count), then
// adds 1.  Epochs grow by one per call (0 is never one) and the last arrival of a call clears the
// word, so the max finds a smaller epoch there.  Each arrival's max and add are one location's
// modifications in program order, so the call's first operation on the word is a max and every
// add lands on a word that carries this call's epoch: one round trip, no retries.  (With the add
// alone, every arrival of a call could land on the stale word before any had replaced it, and
// all of them then retried in turn: 16 arrivals per group took ~16 us.)  A word that still does
// not carry the epoch (garbage with a larger one: the workspace is never cleared) gets (epoch, 1)
// by compare-and-swap; an arrival whose add landed on such a word retries the same way, so stale
// adds are never counted.  Every failed swap means another arrival changed the word, so the loop
// ends after at most `total` rounds.  (The low half would carry into the epoch only from a count
// of 2^32 - 1, which no call reaches.)
// In the forms without a prologue the max goes out at the workgroup's start instead
// (install_epoch; lifted = true here): the arrival is then the add alone, ~1 us shorter with 16
// arrivals per group.  (In the fused forms an early max would hold up the prologue's first wait
// for its loads, which the in-order counter makes wait for the max too.)
__device__ __forceinline__ void install_epoch(uint64_t *ctr, uint32_t epoch) {
  atomicMax(reinterpret_cast<unsigned long long *>(ctr),
            static_cast<unsigned long long>(epoch) << 32);
}
__device__ __forceinline__ bool arrive_last(uint64_t *ctr, uint32_t epoch, uint32_t total,
                                            bool lifted) {
  unsigned long long *p = reinterpret_cast<unsigned long long *>(ctr);
  if (!lifted) install_epoch(ctr, epoch);
  const unsigned long long old = atomicAdd(p, 1ull);
  if (static_cast<uint32_t>(old >> 32) == epoch) return static_cast<uint32_t>(old) + 1u == total;
  unsigned long long cur = old + 1ull;  // a guess; the swap returns the word's actual value
  for (;;) {
    const unsigned long long want = static_cast<uint32_t>(cur >> 32) == epoch
                                        ? cur + 1ull
                                        : (static_cast<unsigned long long>(epoch) << 32) | 1ull;
    const unsigned long long seen = atomicCAS(p, cur, want);
    if (seen == cur) return static_cast<uint32_t>(want) == total;
    cur = seen;
  }
}
// The last arrival clears the word: a replay of the same call (a captured graph, same epoch)
// then starts from a word whose epoch (0) is never a call's.
__device__ __forceinline__ void clear_counter(uint64_t *ctr) {
  atomicExch(reinterpret_cast<unsigned long long *>(ctr), 0ull);
}

template <typename KT, int D, int G, int NW, bool FUSED>
struct DecodeSmem {
  static constexpr int TPL = Vec<KT>::N;
  static constexpr int WT = 64 * TPL;
  static constexpr int NWORD = D / 32;
  // prologue region (fused fp32 storage only, whose projection runs on the VALU): P and the raw
  // rows (G queries + the new key); the bf16 projection takes its operands from registers
  static constexpr bool VPRO = FUSED && sizeof(KT) == 4;
  static constexpr int PRO = VPRO ? (D * D + (G + 1) * D) * 4 : 0;
  // main region: softmax numerators [wave][token][head], reused for the wave merge
  static constexpr int MAIN = NW * WT * G * 4;
  static constexpr int BIG = PRO > MAIN ? PRO : MAIN;
  // persistent small arrays; the walk list has at most D + 24 entries (16 speculative rows, the
  // rest of the union, padding to whole batches)
  static constexpr int NL = D + 24;
  static constexpr int OFF_DL = BIG;                                     // int   [NL]
  static constexpr int OFF_QW = OFF_DL + NL * 4;                         // float [NL][G]
  static constexpr int OFF_QP = OFF_QW + NL * G * 4;                     // float [G+1][D]
  static constexpr int OFF_MW = OFF_QP + (FUSED ? (G + 1) * D * 4 : 0);  // uint  [G][NWORD]
  static constexpr int OFF_KN = OFF_MW + G * NWORD * 4;                  // float [D] new K'
  static constexpr int OFF_VN = OFF_KN + (FUSED ? D * 4 : 0);            // float [D] new V
  static constexpr int OFF_WM = OFF_VN + (FUSED ? D * 4 : 0);            // float [NW][G]
  static constexpr int OFF_WL = OFF_WM + NW * G * 4;                     // float [NW][G]
  static constexpr int OFF_ML = OFF_WL + NW * G * 4;                     // float [2][G]
  static constexpr int BYTES = OFF_ML + 2 * G * 4 + 16;
};

// Merging split partials (m, l, o), written by other workgroups, possibly on other XCDs, so read
// past the non-coherent caches.  merge_partials combines `count` partials of each of the group's
// heads, at split slots first, first + stride, ...: a thread merges EB of its output elements
// side by side, CP splits per batch of loads, so that a merge costs a few memory round trips
// rather than one per split.  dst < 0: the result goes to the output (and its (M, L) to s_M,
// s_L); dst >= 0: it is stored back as a partial in slot dst (an intermediate level; slot dst may
// be one of those read, so every read is done before the first store).
template <int D, int G, int NT>
__device__ void merge_partials(const DecodeArgs &a, size_t head0, int first, int count,
                               int stride, int dst, float *s_M, float *s_L) {
  constexpr int EPT = (G * D + NT - 1) / NT;  // output elements per thread
  constexpr int EB = EPT < 2 ? EPT : 2;
  constexpr int NIT = (EPT + EB - 1) / EB;
  constexpr int CP = 16;
  float rM[NIT][EB], rL[NIT][EB], rO[NIT][EB];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e0 = threadIdx.x + it * EB * NT;
    int dd[EB];
    const float *part[EB];
    float M[EB], O[EB], L[EB];
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int e = min(e0 + j * NT, G * D - 1);  // past the end: a copy of the last, unstored
      const int h = e / D;
      dd[j] = e - h * D;
      part[j] = a.partials + (head0 + h) * a.S * (D + 2);
      M[j] = -INFINITY;
      O[j] = 0.0f;
      L[j] = 0.0f;
    }
    for (int c0 = 0; c0 < count; c0 += CP) {  // running (M, L, O) over batches of CP partials
      float ms[EB][CP], ls[EB][CP], os[EB][CP];
#pragma unroll
      for (int j = 0; j < EB; ++j)
#pragma unroll
        for (int c = 0; c < CP; ++c) {
          // past the last partial: re-read it, weight 0
          const int sp = first + min(c0 + c, count - 1) * stride;
          ms[j][c] = coherent_load(part[j] + sp * (D + 2));
          ls[j][c] = coherent_load(part[j] + sp * (D + 2) + 1);
          os[j][c] = coherent_load(part[j] + sp * (D + 2) + 2 + dd[j]);
        }
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        float Mc = M[j];
#pragma unroll
        for (int c = 0; c < CP; ++c)
          if (c0 + c < count) Mc = fmaxf(Mc, ms[j][c]);
        const float rs = (M[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M[j] - Mc);
        O[j] *= rs;
        L[j] *= rs;
#pragma unroll
        for (int c = 0; c < CP; ++c) {
          const float al = (c0 + c >= count || ms[j][c] == -INFINITY)
                               ? 0.0f
                               : __builtin_amdgcn_exp2f(ms[j][c] - Mc);
          L[j] = fmaf(al, ls[j][c], L[j]);
          O[j] = fmaf(al, os[j][c], O[j]);
        }
        M[j] = Mc;
      }
    }
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      rM[it][j] = M[j];
      rL[it][j] = L[j];
      rO[it][j] = O[j];
    }
  }
  if (dst >= 0) __syncthreads();  // every read of the slots is done (dst is uniform)
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int e = threadIdx.x + it * EB * NT + j * NT;
      if (e >= G * D) continue;
      const int h = e / D, dd = e - h * D;
      if (dst < 0) {
        a.out[(head0 + h) * D + dd] = rO[it][j] / rL[it][j];
        if (dd == 0) {
          s_M[h] = rM[it][j];
          s_L[h] = rL[it][j];
        }
      } else {
        float *part = a.partials + ((head0 + h) * a.S + dst) * (D + 2);
        if (dd == 0) {
          publish(part + 0, rM[it][j]);
          publish(part + 1, rL[it][j]);
        }
        publish(part + 2 + dd, rO[it][j]);
      }
    }
}

// The last workgroup of a (b, g): merge the group's partials (count of them, at slots 0,
// stride, 2 stride, ...) into the output and, in mass mode, add every token's normalised
// probability (summed over the group's heads) to its mass (slot `restart`, if any, starts again
// from 0); then reset the group's counter.
template <int D, int G, int NT>
__device__ void merge_splits(const DecodeArgs &a, size_t head0, int bg, float *s_M, float *s_L,
                             int restart, int count, int stride) {
  constexpr int CH = 8;
  // mass mode: the first batch of scores and masses is loaded before the partials, so that the
  // two sets of round trips overlap
  float *mass = a.mass ? a.mass + static_cast<size_t>(bg) * a.T_cap : nullptr;
  float sc[CH][G], mv[CH];
  auto load_batch = [&](int t0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int t = min(t0 + c * NT, a.len - 1);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[c][h] = coherent_load(a.scores + (head0 + h) * a.T_cap + t);
      mv[c] = mass[t];
    }
  };
  if (mass) load_batch(threadIdx.x);
  merge_partials<D, G, NT>(a, head0, 0, count, stride, -1, s_M, s_L);
  if (mass) {
    __syncthreads();
    for (int t0 = threadIdx.x; t0 < a.len; t0 += NT * CH) {
      if (t0 != static_cast<int>(threadIdx.x)) load_batch(t0);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int t = t0 + c * NT;
        if (t < a.len) {
          float add = 0.0f;
#pragma unroll
          for (int h = 0; h < G; ++h) add += __builtin_amdgcn_exp2f(sc[c][h] - s_M[h]) / s_L[h];
          mass[t] = (t == restart ? 0.0f : mv[c]) + add;  // a restarted slot's mass begins at 0
        }
      }
    }
  }
  if (threadIdx.x == 0) clear_counter(&a.counters[bg]);
}

// Past kMergeFan * 2 splits per group the merge takes two levels: the last workgroup of each run
// of kMergeFan consecutive splits (a counter per run) merges the run into its first slot, and the
// last of those merges the runs' results.  Both levels are one round of loads, and the first
// overlaps with the workgroups still streaming.

// Ends a split's work once its partials are published: the group's last workgroup merges.
// Returns in every workgroup; s_last is a workgroup-shared flag.
template <int D, int G, int NT, bool LIFTED>
__device__ __forceinline__ void finish_split(const DecodeArgs &a, size_t head0, int bg,
                                             int split, int *s_last, float *s_M, float *s_L,
                                             int restart) {
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partials, scores and cache writes have landed
  __syncthreads();
  if (a.S > 2 * kMergeFan) {
    const int run = split / kMergeFan, first = run * kMergeFan;
    const int cnt = min(kMergeFan, a.S - first);
    const int nrun = (a.S + kMergeFan - 1) / kMergeFan;
    uint64_t *rc = a.run_counters + static_cast<size_t>(bg) * a.run_stride + run;
    if (tid == 0) *s_last = arrive_last(rc, a.epoch, static_cast<uint32_t>(cnt), LIFTED);
    __syncthreads();
    if (!*s_last) return;
    merge_partials<D, G, NT>(a, head0, first, cnt, 1, first, s_M, s_L);
    if (tid == 0) clear_counter(rc);
    __builtin_amdgcn_s_waitcnt(0);  // the run's result has landed
    __syncthreads();
    if (tid == 0)
      *s_last = arrive_last(&a.counters[bg], a.epoch, static_cast<uint32_t>(nrun), LIFTED);
    __syncthreads();
    if (!*s_last) return;
    merge_splits<D, G, NT>(a, head0, bg, s_M, s_L, restart, nrun, kMergeFan);
    return;
  }
  if (tid == 0)
    *s_last = arrive_last(&a.counters[bg], a.epoch, static_cast<uint32_t>(a.S), LIFTED);
  __syncthreads();
  if (!*s_last) return;
  merge_splits<D, G, NT>(a, head0, bg, s_M, s_L, restart, a.S, 1);
}

template <typename KT, int D, int G, int NT>
__device__ __forceinline__ void select_group_heads(const DecodeArgs &a, size_t head0,
                                                   bool with_key, bool split0, float (*s_qp)[D],
                                                   uint32_t (*s_mw)[D / 32], float *s_knew);

// Fused prologue shared by the fused decode step and the fused H2O step, fp32 storage: stage P in LDS, project
// the group's G query rows and, when with_key, the new token's key (q'_h[i] = sum_j q_h[j] P[j][i]
// in fp32, j ascending: the arithmetic of select_kernel and of the key projection, so the results
// are those of the separate calls bit for bit), keep the key's stored (rounded) K' and raw V in
// LDS, and select every head's top-k dims into mask words.  split0 writes q_proj_out / mask_out.
// LDS: sP [D][D], sq [G+1][D], s_qp [G+1][D], s_mw [G][D/32], s_knew and s_vnew [D].
// after_staging() runs once P and the rows are on their way to LDS (the caller issues its own
// loads there; the barriers here order LDS only, so those loads stay in flight).  Ends with a
// workgroup barrier.
template <typename KT, int D, int G, int NT, typename F>
__device__ __forceinline__ void fused_project_select(const DecodeArgs &a, size_t head0, int bg,
                                                     bool with_key, bool split0, float *sP,
                                                     float (*sq)[D], float (*s_qp)[D],
                                                     uint32_t (*s_mw)[D / 32], float *s_knew,
                                                     float *s_vnew, F &&after_staging) {
  constexpr int NWORD = D / 32;
  constexpr int E = D / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // the raw rows' loads first, so that they are in flight with P's; then the LDS stores
  constexpr int QPT = (G * D + NT - 1) / NT;  // raw query elements per thread
  constexpr int NV = D * D / (NT * 4);        // 16-byte pieces of P per thread
  const KT *qr = static_cast<const KT *>(a.q_raw) + head0 * D;
  const size_t at = static_cast<size_t>(bg) * D + min(tid, D - 1);
  float qv[QPT];
#pragma unroll
  for (int r = 0; r < QPT; ++r) qv[r] = load_elem<KT>(qr + min(tid + r * NT, G * D - 1));
  const float kn = load_elem<KT>(static_cast<const KT *>(a.k_new) + at);
  const float vn = load_elem<KT>(static_cast<const KT *>(a.v_new) + at);
  constexpr int CH = NV < 16 ? NV : 16;  // P pieces per batch of loads
#pragma unroll
  for (int v0 = 0; v0 < NV; v0 += CH) {
    float4 st[CH];
#pragma unroll
    for (int v = 0; v < CH; ++v)
      st[v] = *reinterpret_cast<const float4 *>(&a.P[((v0 + v) * NT + tid) * 4]);
#pragma unroll
    for (int v = 0; v < CH; ++v)
      *reinterpret_cast<float4 *>(&sP[((v0 + v) * NT + tid) * 4]) = st[v];
  }
#pragma unroll
  for (int r = 0; r < QPT; ++r)
    if (tid + r * NT < G * D) sq[(tid + r * NT) / D][(tid + r * NT) % D] = qv[r];
  if (with_key && tid < D) {
    sq[G][tid] = kn;
    s_vnew[tid] = vn;
  }
  after_staging();  // the caller's loads go out while the projection runs
  lds_barrier();
  // q'_h[i] = sum_j q_h[j] P[j][i] (fp32, j ascending); thread -> dim i, rows r0, r0+NT/D, ...
  // The j loop is fully unrolled and branch-free (rows past the last are computed on a
  // clamped row and discarded), so the LDS reads of later j are issued ahead of the fmas.
  {
    constexpr int RSTEP = NT / D;
    constexpr int RPT = (G + 1 + RSTEP - 1) / RSTEP;
    const int nrows = G + (with_key ? 1 : 0);
    const int i = tid % D, r0 = tid / D;
    float acc[RPT];
    int row[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      acc[r] = 0.0f;
      row[r] = min(r0 + r * RSTEP, G);
    }
#pragma unroll 8
    for (int j = 0; j < D; j += 4) {
      float p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) p[c] = sP[(j + c) * D + i];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const float4 q4 = *reinterpret_cast<const float4 *>(&sq[row[r]][j]);  // broadcast
        acc[r] = fmaf(q4.x, p[0], acc[r]);
        acc[r] = fmaf(q4.y, p[1], acc[r]);
        acc[r] = fmaf(q4.z, p[2], acc[r]);
        acc[r] = fmaf(q4.w, p[3], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      if (r0 + r * RSTEP < nrows) s_qp[r0 + r * RSTEP][i] = acc[r];
  }
  lds_barrier();
  select_group_heads<KT, D, G, NT>(a, head0, with_key, split0, s_qp, s_mw, s_knew);
}

// The fused prologue after the projection: the new key's stored K' (rounded once) into s_knew,
// every head's top-k dims of its q' (s_qp rows 0 .. G-1) into mask words; split0 writes
// q_proj_out / mask_out.  Ends with a workgroup barrier.
template <typename KT, int D, int G, int NT>
__device__ __forceinline__ void select_group_heads(const DecodeArgs &a, size_t head0,
                                                   bool with_key, bool split0, float (*s_qp)[D],
                                                   uint32_t (*s_mw)[D / 32], float *s_knew) {
  constexpr int NWORD = D / 32;
  constexpr int E = D / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (with_key && tid < D) {
    // the new token's K' as it will be stored (rounded once); the caller writes it to the cache
    // only after its own reads of that column are done
    const KT kq = store_elem<KT>(s_qp[G][tid]);
    s_knew[tid] = load_elem<KT>(&kq);
  }
  for (int h = w; h < G; h += NT / 64) {
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = s_qp[h][lane + 64 * e];
    bool sel[E];
    wave_topk_threshold<E>(x, a.d_sel, a.k, sel);
    uint64_t sb[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sb[e] = __ballot(sel[e]);
    if (lane < NWORD) {
      const uint64_t bb = (lane >> 1) ? sb[E - 1] : sb[0];
      const uint32_t word =
          (lane & 1) ? static_cast<uint32_t>(bb >> 32) : static_cast<uint32_t>(bb);
      s_mw[h][lane] = word;
      if (split0 && a.mask_out) a.mask_out[(head0 + h) * NWORD + lane] = word;
    }
    if (split0 && a.q_proj_out) {
#pragma unroll
      for (int e = 0; e < E; ++e) a.q_proj_out[(head0 + h) * D + lane + 64 * e] = x[e];
    }
  }
  lds_barrier();
}

// Fused prologue, bf16 storage: the group's G raw query rows and the new key projected on MFMA
// (proj_mfma: the arithmetic of aqua_select_dims and aqua_project_keys for bf16, so q', the masks
// and the stored K' are those of the separate calls bit for bit), then select_group_heads.  The
// A operand is 16 rows: the G queries, the new key at row G, and the key again past it (those
// rows are discarded).  Wavefront w computes column blocks w, w + NW, ...  ALL: the loads of every
// block's values of P are issued before after_loads() (the caller issues its own loads there, and
// they stay in flight through the projection and the selection: the waits for P's values leave
// them outstanding); otherwise the blocks go one at a time, each load followed by its use, for
// fewer live registers.  after_proj() runs once the projection is done (more of the caller's
// loads: issued up front as well, they would stall the prologue's instructions behind a full
// memory pipeline).  LDS: s_qp [G+1][D],
// s_mw [G][D/32], s_knew and s_vnew [D].  Ends with a workgroup barrier.
template <int D, int G, int NT, bool ALL, typename F, typename F2>
__device__ __forceinline__ void fused_project_select_mfma(const DecodeArgs &a, size_t head0,
                                                          int bg, bool with_key, bool split0,
                                                          float (*s_qp)[D],
                                                          uint32_t (*s_mw)[D / 32],
                                                          float *s_knew, float *s_vnew,
                                                          F &&after_loads, F2 &&after_proj) {
  constexpr int KS = D / 32, NB = D / 16, NW = NT / 64;
  constexpr int BPW = (NB + NW - 1) / NW;  // column blocks per wavefront
  static_assert(G + 1 <= 16, "queries and key fit one 16-row A operand");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15;
  const bf16_t *row = r < G ? static_cast<const bf16_t *>(a.q_raw) + (head0 + r) * D
                            : static_cast<const bf16_t *>(a.k_new) + static_cast<size_t>(bg) * D;
  u32x4_t av[KS];
  load_a_row<KS>(row, av);
  const float vn = load_elem<bf16_t>(static_cast<const bf16_t *>(a.v_new) +
                                     static_cast<size_t>(bg) * D + min(tid, D - 1));
  auto store_tile = [&](int blk, const f32x4_t &x) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int orow = 4 * (lane >> 4) + rr;
      if (orow <= G) s_qp[orow][16 * blk + (lane & 15)] = x[rr];
    }
  };
  if constexpr (ALL) {
    float pv[BPW][KS][8];
#pragma unroll
    for (int i = 0; i < BPW; ++i) load_p_raw<KS>(a.P, 16 * min(w + i * NW, NB - 1), pv[i]);
    __builtin_amdgcn_sched_barrier(0);  // P's loads are issued before the caller's
    after_loads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      PParts<KS> pp;
      split_p_parts<KS>(pv[i], pp);
      if (w + i * NW < NB) store_tile(w + i * NW, proj_mfma<KS>(av, pp));  // uniform
    }
  } else {
    after_loads();
    for (int blk = w; blk < NB; blk += NW) {
      PParts<KS> pp;
      load_p_parts<KS>(a.P, 16 * blk, pp);
      store_tile(blk, proj_mfma<KS>(av, pp));
    }
  }
  if (with_key && tid < D) s_vnew[tid] = vn;
  after_proj();
  lds_barrier();
  select_group_heads<bf16_t, D, G, NT>(a, head0, with_key, split0, s_qp, s_mw, s_knew);
}

// Two workgroups share each CU, and the issue arbiter favours older wavefronts: left alone, the
// first workgroup on a CU streams its rows faster and finishes early, and the CU runs the rest
// of the launch half occupied.  Each wavefront therefore lowers its priority as it progresses
// (3 in its first quarter of batches, 0 in its last), so that the one behind is served first.
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int q = total > 0 ? (4 * done) / total : 3;
  if (q <= 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 1) __builtin_amdgcn_s_setprio(2);
  else if (q == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// At least two waves per SIMD must stay resident (the decode streams at full bandwidth only
// then): at most 256 VGPRs.  Wavefronts per workgroup (decode_layout): 4; for G = 4 and G = 8,
// 8 when that still gives at least one workgroup per CU: one 512-thread workgroup per CU, whose
// wavefronts are all of one age (with two 4-wavefront workgroups per CU the second one resident
// ran ~4 us behind the first; 8 measured 1 us faster on the 16 x 8-group, 8192-token decode, but
// halves the grid, and a 32-workgroup grid at 16384 tokens and batch 1 ran 48 against 35 us).
// G = 8 doubles the LDS numerators per wavefront (77 KB per 4-wavefront workgroup, 143 KB per
// 8-wavefront one in bf16), which still leaves two wavefronts per SIMD.
template <typename KT, int D, int G, int NW, bool FUSED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(DecodeArgs a) {
  using SM = DecodeSmem<KT, D, G, NW, FUSED>;
  constexpr int TPL = SM::TPL;     // tokens per lane per K' row load
  constexpr int WT = SM::WT;       // tokens per wavefront
  constexpr int EPL = Vec<KT>::N;  // V elements per lane per load
  constexpr int LPT = D / EPL;     // lanes per V row
  static_assert(LPT >= 8, "the V rows' lane butterfly starts at lane ^ 8");
  constexpr int TPI = 64 / LPT;    // V rows per wavefront load
  constexpr int NWORD = SM::NWORD;
  constexpr int NT = NW * 64;
  constexpr int E = D / 64;        // dims per lane in the top-k
  constexpr int SPLIT = NW * WT;   // tokens per workgroup
  static_assert(WT % (TPI * kUnroll) == 0, "V loop tiling");
  static_assert(D <= WT, "LDS reuse of the numerator buffer for the wave merge");

  __shared__ __align__(16) unsigned char smem[SM::BYTES];
  int *s_dl = reinterpret_cast<int *>(smem + SM::OFF_DL);
  float(*s_qw)[G] = reinterpret_cast<float(*)[G]>(smem + SM::OFF_QW);
  float(*s_qp)[D] = reinterpret_cast<float(*)[D]>(smem + SM::OFF_QP);
  uint32_t(*s_mw)[NWORD] = reinterpret_cast<uint32_t(*)[NWORD]>(smem + SM::OFF_MW);
  float *s_knew = reinterpret_cast<float *>(smem + SM::OFF_KN);
  float *s_vnew = reinterpret_cast<float *>(smem + SM::OFF_VN);
  float(*s_wm)[G] = reinterpret_cast<float(*)[G]>(smem + SM::OFF_WM);
  float(*s_wl)[G] = reinterpret_cast<float(*)[G]>(smem + SM::OFF_WL);
  float *s_M = reinterpret_cast<float *>(smem + SM::OFF_ML);
  float *s_L = s_M + G;
  __shared__ int s_last;

  // Every kernel argument this workgroup uses is read here, in one batch: left to the compiler,
  // the reads go out one dependent round trip at a time, ~1 us each before the first HBM load.
  asm volatile("" ::"s"(a.kp), "s"(a.v), "s"(a.q_proj), "s"(a.mask), "s"(a.q_raw), "s"(a.k_new),
               "s"(a.P), "s"(a.partials), "s"(a.Hq), "s"(a.Hkv), "s"(a.d_store), "s"(a.T_cap),
               "s"(a.len), "s"(a.S), "s"(a.qscale), "s"(a.d_sel), "s"(a.k), "s"(a.B),
               "s"(a.tail_last));
  // Grid (split, KV head, batch): the linear workgroup index (the one the dispatcher deals to
  // the XCDs in turn) is split + S (g + Hkv b).  With tail_last (set where the grid takes more
  // than one round of resident workgroups and the last split of each group is partial) that
  // index is dealt differently: first the S - 1 full splits of every group, group by group,
  // then every group's last split, so that the first round runs full splits only and the
  // short ones follow, instead of holding slots while full splits wait for the next round.
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int split = blockIdx.x, bg = blockIdx.z * a.Hkv + blockIdx.y;
  if (a.tail_last) {
    const int lin = bg * a.S + split, nfull = (a.S - 1) * a.B * a.Hkv;
    if (lin < nfull) {
      bg = lin / (a.S - 1);
      split = lin - bg * (a.S - 1);
    } else {
      bg = lin - nfull;
      split = a.S - 1;
    }
  }
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int wg_lin = bg * a.S + split;
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(g) * G;
  // Fused: the cache holds len - 1 tokens, the new one is position len - 1.
  const int len_c = FUSED ? a.len - 1 : a.len;
  const bool owner = FUSED && split == (a.len - 1) / SPLIT;

  // This wavefront's tokens.  Lanes past the cached length read the last valid 16-byte chunk
  // instead (same cache line as a live lane); their scores are discarded below.
  const int tw0 = split * SPLIT + w * WT;
  const int tl = tw0 + lane * TPL;
  const bool wave_live = tw0 < len_c;
  const int tl_ld = len_c > 0 ? min(tl, ((len_c - 1) / TPL) * TPL) : 0;
  const KT *kbase = static_cast<const KT *>(a.kp) +
                    static_cast<size_t>(bg) * a.d_store * a.T_cap + tl_ld;
  // Each workgroup starts its walk over the K' rows at its own offset, so that workgroups running
  // at the same time read different rows (rows of one group are T_cap apart, and a lock-step walk
  // would send every workgroup to the same few HBM channels).  The offset mixes in the higher
  // bits of the workgroup index: with many splits per group (a long context at batch 1)
  // workgroups 16 apart would otherwise start on the same batch (measured at 131072 tokens:
  // 106 us with the plain multiple, 97 us mixed; unchanged at batch 16).
  const int wg_mix = (wg_lin * 5) ^ (wg_lin >> 4);
  if (!FUSED && tid == 0) {  // this call's epoch into the counters the workgroup arrives at
    install_epoch(&a.counters[bg], a.epoch);
    if (a.S > 2 * kMergeFan)
      install_epoch(a.run_counters + static_cast<size_t>(bg) * a.run_stride + split / kMergeFan,
                    a.epoch);
  }

  // Fused, bf16 storage: the first two batches of K' rows are requested before the prologue,
  // speculatively, so that HBM is busy while the queries are projected and selected.  They are a
  // cyclic run of 16 of the lowest spec_w stored dims (spec_w: the largest power of two up to
  // 32 and d_store, so that the run wraps with a mask), which the selection nearly always keeps
  // (the offline projection orders its dims by decreasing importance); a speculative row no head
  // kept is weighted 0.  The walk then goes on over the rest of the union.  (Not for G = 8: the
  // registers the speculative rows hold would spill there.)
  constexpr bool SPEC = FUSED && sizeof(KT) == 2 && NW >= 4 && G <= 4;
  constexpr int NSPEC = SPEC ? 2 * kUnroll : 0;
  const int spec_w = a.d_store >= 32 ? 32 : 1 << (31 - __clz(a.d_store));
  const int spec_r0 = wg_mix & (spec_w - 1);
  const int spec_n = min(NSPEC, spec_w);  // distinct speculative rows
  uint4 kA[kUnroll], kB[kUnroll];

  // V rows of this wavefront's tokens: lane -> row sub of each group of TPI, elements cl * EPL..
  const int sub = lane / LPT, cl = lane - sub * LPT;
  const int nrow = min(WT, len_c - tw0);  // may be <= 0
  const KT *vbase = static_cast<const KT *>(a.v) +
                    (static_cast<size_t>(bg) * a.T_cap + tw0) * D + cl * EPL;
  // With the speculative rows, the fused prologue also requests this wavefront's first batch of
  // V rows (which no selection decides) and holds it in registers until the V pass, so that HBM
  // stays busy through the projection and the selection.  (Copies straight into LDS would free
  // the registers, but the compiler then waits for every outstanding load at each wait while
  // they are in flight.)
  constexpr bool VPRE = SPEC;
  uint4 vC[VPRE ? kUnroll : 1];
  auto v_prefetch = [&] {
    if constexpr (VPRE) {
      // rows past the cached length read the last cached row (their p is 0); a wavefront past
      // the end reads a valid row too, so that every wavefront issues the same loads
      const int last = len_c > 0 ? len_c - 1 : 0;
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
        const int tok = min(tw0 + i * TPI + sub, last);
        vC[i] = load16(static_cast<const KT *>(a.v) +
                       (static_cast<size_t>(bg) * a.T_cap + tok) * D + cl * EPL);
      }
    }
  };

  // ---- fused prologue: project the group's queries (and the new key), select their dims
  if constexpr (FUSED) {
    if constexpr (SPEC) {
      // The speculative loads go out in three parts, one batch each: at the start, after the
      // projection, and after the selection.  All at once they would fill the memory pipeline
      // (a CU holds about 8 KB of loads per wavefront in flight), and every instruction of the
      // prologue behind them would wait for room to issue them.  Unconditional (a wavefront
      // past the cached tokens reads its clamped, valid addresses): loads issued under a branch
      // would make every later wait count them as possibly absent, i.e. wait for all of them.
      fused_project_select_mfma<D, G, NT, true>(
          a, head0, bg, owner, split == 0, s_qp, s_mw, s_knew, s_vnew,
          [&] {
#pragma unroll
            for (int i = 0; i < kUnroll; ++i)
              kA[i] = load16(kbase + static_cast<size_t>((spec_r0 + i) & (spec_w - 1)) * a.T_cap);
          },
          [&] {
#pragma unroll
            for (int i = 0; i < kUnroll; ++i)
              kB[i] = load16(kbase + static_cast<size_t>((spec_r0 + kUnroll + i) & (spec_w - 1)) *
                                         a.T_cap);
          });
      v_prefetch();
    } else if constexpr (sizeof(KT) == 2) {
      fused_project_select_mfma<D, G, NT, false>(a, head0, bg, owner, split == 0, s_qp, s_mw,
                                                 s_knew, s_vnew, [] {}, [] {});
    } else {
      fused_project_select<KT, D, G, NT>(a, head0, bg, owner, split == 0,
                                         reinterpret_cast<float *>(smem),
                                         reinterpret_cast<float(*)[D]>(smem + D * D * 4), s_qp,
                                         s_mw, s_knew, s_vnew, [] {});
    }
  }

  // ---- the walk list: the speculative rows (fused bf16), then the union U of the group's masks
  // (restricted to stored dims) less those rows, padded to whole batches with a dim at zero
  // weight (re-reads hit in cache).  Entry e: dim s_dl[e], head weights s_qw[e][h] =
  // q'_h[dim] * scale * log2 e where head h selected dim, else 0.  Uniform per workgroup.
  auto mask_word = [&](int h, int wd) -> uint32_t {
    if constexpr (FUSED) return s_mw[h][wd];
    else return a.mask[(head0 + h) * NWORD + wd];
  };
  auto q_val = [&](int h, int dim) -> float {
    if constexpr (FUSED) return s_qp[h][dim];
    else return a.q_proj[(head0 + h) * D + dim];
  };
  uint32_t R[NWORD];
  int nR = 0, last_dim = 0;
#pragma unroll
  for (int wd = 0; wd < NWORD; ++wd) {
    uint32_t u = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) u |= mask_word(h, wd);
    const int lo = wd * 32;
    if (a.d_store <= lo) u = 0;
    else if (a.d_store < lo + 32) u &= (1u << (a.d_store - lo)) - 1u;
    if (SPEC && wd == 0) {  // the speculative rows lie in dims 0..31: spec_n of them, cyclic
      const uint64_t run = ((spec_n >= 32 ? 0xffffffffull : ((1ull << spec_n) - 1)) << spec_r0);
      const uint32_t wmask = spec_w >= 32 ? 0xffffffffu : (1u << spec_w) - 1u;
      const uint32_t sp = (static_cast<uint32_t>(run) | static_cast<uint32_t>(run >> spec_w)) & wmask;
      u &= ~sp;
    }
    R[wd] = u;
    nR += __popc(u);
    if (u) last_dim = lo + 31 - __clz(u);
  }
  const int nRp = (nR + kUnroll - 1) / kUnroll * kUnroll;
  if (SPEC && tid < NSPEC) {
    // speculative entry tid: dim (r0 + tid) mod spec_w; entries past the distinct ones weigh 0
    const int dim = (spec_r0 + tid) & (spec_w - 1);
    s_dl[tid] = dim;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool keep = tid < spec_n && ((mask_word(h, dim >> 5) >> (dim & 31)) & 1u);
      s_qw[tid][h] = keep ? q_val(h, dim) * a.qscale : 0.0f;
    }
  }
  if (tid < D) {
    const int wd = tid >> 5, bit = tid & 31;
    // this dim's mask bits and q' for every head, read before they are known to be needed (in
    // the plain form they are global loads: one round trip with the union's)
    uint32_t mw[G];
    float qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mw[h] = mask_word(h, wd);
      qv[h] = q_val(h, tid);
    }
    uint32_t rw = 0;
    int pos = 0;
#pragma unroll
    for (int x = 0; x < NWORD; ++x) {
      if (x < wd) pos += __popc(R[x]);
      if (x == wd) rw = R[x];
    }
    pos += __popc(rw & ((1u << bit) - 1u));
    const int nb = nRp / kUnroll;
    const int rot = nb ? (wg_mix % nb) * kUnroll : 0;
    if ((rw >> bit) & 1u) {
      const int at = NSPEC + (pos + nRp - rot) % nRp;
      s_dl[at] = tid;
#pragma unroll
      for (int h = 0; h < G; ++h) s_qw[at][h] = ((mw[h] >> bit) & 1u) ? qv[h] * a.qscale : 0.0f;
    }
    if (tid >= nR && tid < nRp) {
      const int at = NSPEC + (tid + nRp - rot) % nRp;
      s_dl[at] = last_dim;
#pragma unroll
      for (int h = 0; h < G; ++h) s_qw[at][h] = 0.0f;
    }
  }
  // LDS only: the speculative loads stay in flight
  lds_barrier();

  // ---- phase 1: log2-domain scores of this wavefront's cached tokens
  float acc[G][TPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < TPL; ++j) acc[h][j] = 0.0f;

  // Software pipeline over batches of kUnroll rows, two register sets A and B in turn, with a
  // batch in flight during the arithmetic of the one before; the last batches are peeled off so
  // that nothing is fetched past the end (a re-read there would go back to memory: the loads are
  // non-temporal).
#define AQUA_K_LOAD(BUF, BATCH)                                                          \
  _Pragma("unroll") for (int i = 0; i < kUnroll; ++i) BUF[i] = load16(                   \
      kbase + static_cast<size_t>(s_dl[(BATCH) * kUnroll + i]) * a.T_cap)
#define AQUA_K_FMA(BUF, BATCH)                                                           \
  _Pragma("unroll") for (int i = 0; i < kUnroll; ++i) {                                  \
    float kv[TPL];                                                                        \
    Vec<KT>::unpack(BUF[i], kv);                                                          \
    float qw[G];                                                                          \
    _Pragma("unroll") for (int h = 0; h < G; ++h) qw[h] = s_qw[(BATCH) * kUnroll + i][h]; \
    _Pragma("unroll") for (int h = 0; h < G; ++h)                                        \
        _Pragma("unroll") for (int j = 0; j < TPL; ++j) acc[h][j] =                       \
        fmaf(qw[h], kv[j], acc[h][j]);                                                    \
  }
  const int nbat = (NSPEC + nRp) / kUnroll;
  const int ptot = nbat + WT / (TPI * kUnroll);
  if (wave_live && nbat > 0) {
    int bi = 0;
    if constexpr (SPEC) {
      // batches 0 and 1 are in flight already: each batch's loads go out two batches ahead
      for (; bi + 3 < nbat; bi += 2) {
        progress_priority(bi, ptot);
        AQUA_K_FMA(kA, bi);
        AQUA_K_LOAD(kA, bi + 2);
        __builtin_amdgcn_sched_barrier(0);
        AQUA_K_FMA(kB, bi + 1);
        AQUA_K_LOAD(kB, bi + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the last one to three batches (bi .. nbat - 1): nothing fetched past the end
      progress_priority(bi, ptot);
      const int left = nbat - bi;
      AQUA_K_FMA(kA, bi);
      if (left == 3) AQUA_K_LOAD(kA, bi + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (left >= 2) AQUA_K_FMA(kB, bi + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (left == 3) AQUA_K_FMA(kA, bi + 2);
    } else {
      // the loads of batch i + 1 are issued before the arithmetic of batch i; inside the loop
      // every load is unconditional, so the wait before each batch's arithmetic is exactly "one
      // batch still in flight"
      AQUA_K_LOAD(kA, 0);
      for (; bi + 2 < nbat; bi += 2) {
        progress_priority(bi, ptot);
        AQUA_K_LOAD(kB, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
        AQUA_K_FMA(kA, bi);
        AQUA_K_LOAD(kA, bi + 2);
        __builtin_amdgcn_sched_barrier(0);
        AQUA_K_FMA(kB, bi + 1);
      }
      // the last one or two batches: nothing more to prefetch
      progress_priority(bi, ptot);
      if (bi + 1 < nbat) {
        AQUA_K_LOAD(kB, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
        AQUA_K_FMA(kA, bi);
        __builtin_amdgcn_sched_barrier(0);
        AQUA_K_FMA(kB, bi + 1);
      } else {
        AQUA_K_FMA(kA, bi);
      }
    }
  }
#undef AQUA_K_LOAD
#undef AQUA_K_FMA

  // The V pass's first two batches (batches 1 and 2 when batch 0 came with the prologue) are
  // requested here, before the softmax and the workgroup barrier: they depend on this
  // wavefront's tokens only, and without them nothing would be in flight across that stretch.
  // Rows past the cached length read the last cached row (weight 0), as in the V pass.
  constexpr int RB = TPI * kUnroll;  // V rows per batch
  constexpr int VB0 = VPRE ? 1 : 0;  // first batch requested here
  uint4 vA[kUnroll], vB[kUnroll];
  {
    const int last = len_c > 0 ? len_c - 1 : 0;
    const KT *vg = static_cast<const KT *>(a.v) + static_cast<size_t>(bg) * a.T_cap * D + cl * EPL;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      vA[i] = load16(vg + static_cast<size_t>(min(tw0 + VB0 * RB + i * TPI + sub, last)) * D);
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      vB[i] = load16(vg + static_cast<size_t>(min(tw0 + (VB0 + 1) * RB + i * TPI + sub, last)) * D);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- softmax numerators within the wavefront
#pragma unroll
  for (int j = 0; j < TPL; ++j)
    if (tl + j >= len_c)
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h][j] = -INFINITY;
  // fused: the new token's score (uniform over the wavefront that owns its position), from its
  // K' in LDS; it enters the softmax as one more term next to the cached tokens
  const int off_new = FUSED ? (a.len - 1) - tw0 : -1;
  const bool new_here = FUSED && owner && off_new >= 0 && off_new < WT;
  float s_new[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s_new[h] = -INFINITY;
  if (new_here) {
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.0f;
    for (int u = lane; u < nbat * kUnroll; u += 64) {
      const float kv = s_knew[s_dl[u]];
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = fmaf(s_qw[u][h], kv, part[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s_new[h] = wave_sum(part[h]);
  }
  if (a.mass) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int j = 0; j < TPL; ++j)
        if (tl + j < len_c) publish(a.scores + (head0 + h) * a.T_cap + tl + j, acc[h][j]);
      if (new_here && lane == 0) publish(a.scores + (head0 + h) * a.T_cap + (a.len - 1), s_new[h]);
    }
  }
  float m[G], l[G], p_new[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = acc[h][0];
#pragma unroll
    for (int j = 1; j < TPL; ++j) mx = fmaxf(mx, acc[h][j]);
    m[h] = fmaxf(wave_max(mx), s_new[h]);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      const float p = (m[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(acc[h][j] - m[h]);
      acc[h][j] = p;
      sum += p;
    }
    p_new[h] = new_here ? __builtin_amdgcn_exp2f(s_new[h] - m[h]) : 0.0f;
    l[h] = wave_sum(sum) + p_new[h];
  }
  float *s_p = reinterpret_cast<float *>(smem);
  float *sp = s_p + w * (WT * G);
#pragma unroll
  for (int j = 0; j < TPL; ++j)
#pragma unroll
    for (int h = 0; h < G; ++h) sp[(lane * TPL + j) * G + h] = acc[h][j];
  __syncthreads();
  if (owner && tid < D) {
    // append the new token: every K' load of this workgroup has been consumed by now, and the
    // V pass below never reads row len - 1 (it takes the new V from LDS)
    const size_t col = static_cast<size_t>(a.len - 1);
    if (tid < a.d_store)
      static_cast<KT *>(a.kp_w)[(static_cast<size_t>(bg) * a.d_store + tid) * a.T_cap + col] =
          store_elem<KT>(s_knew[tid]);
    static_cast<KT *>(a.v_w)[(static_cast<size_t>(bg) * a.T_cap + col) * D + tid] =
        store_elem<KT>(s_vnew[tid]);  // exact: s_vnew holds the stored value widened
  }

  // ---- phase 2: o = sum_t p_t V_t over this wavefront's cached tokens
  // Rows past the cached length read the last valid row (their p is 0), to keep loads
  // unconditional.
  float o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
  // same pipeline over batches of RB rows
#define AQUA_V_LOAD(BUF, BATCH)                                                          \
  _Pragma("unroll") for (int i = 0; i < kUnroll; ++i) BUF[i] = load16(                   \
      vbase + static_cast<size_t>(min(min(BATCH, vbat - 1) * RB + i * TPI + sub, nrow - 1)) * D)
#define AQUA_V_FMA(BUF, BATCH)                                                           \
  _Pragma("unroll") for (int i = 0; i < kUnroll; ++i) {                                  \
    const int t = (BATCH) * RB + i * TPI + sub;                                           \
    float vv[EPL];                                                                        \
    Vec<KT>::unpack(BUF[i], vv);                                                          \
    float p[G];                                                                           \
    _Pragma("unroll") for (int h = 0; h < G; ++h) p[h] = sp[t * G + h];                 \
    _Pragma("unroll") for (int h = 0; h < G; ++h)                                        \
        _Pragma("unroll") for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p[h], vv[e], o[h][e]); \
  }
  const int vbat = nrow > 0 ? (nrow + RB - 1) / RB : 0;
  int bi = 0;
  if constexpr (VPRE) {
    // batch 0 came in with the prologue and is added in every wavefront (one with fewer rows
    // reads valid rows again and adds them at p = 0): a use under a branch would let the
    // compiler move the prologue's loads down to it
    AQUA_V_FMA(vC, 0);
    bi = 1;
  }
  // batches bi (vA) and bi + 1 (vB) are in flight; each batch's loads go out two batches ahead
  for (; bi + 3 < vbat; bi += 2) {
    progress_priority(nbat + bi, nbat + WT / (TPI * kUnroll));
    AQUA_V_FMA(vA, bi);
    AQUA_V_LOAD(vA, bi + 2);
    __builtin_amdgcn_sched_barrier(0);
    AQUA_V_FMA(vB, bi + 1);
    AQUA_V_LOAD(vB, bi + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last one to three batches: nothing fetched past the end
  progress_priority(nbat + bi, nbat + WT / (TPI * kUnroll));
  {
    const int left = vbat - bi;
    if (left >= 1) AQUA_V_FMA(vA, bi);
    if (left == 3) AQUA_V_LOAD(vA, bi + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (left >= 2) AQUA_V_FMA(vB, bi + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (left == 3) AQUA_V_FMA(vA, bi + 2);
  }
#undef AQUA_V_LOAD
#undef AQUA_V_FMA
  __builtin_amdgcn_s_setprio(0);
  if (new_here && sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p_new[h], s_vnew[cl * EPL + e], o[h][e]);
  }
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = add_xor(o[h][e], off);
  __syncthreads();  // every wavefront is done with the numerators

  // ---- merge the workgroup's wavefronts, write this split's partials
  float *so = s_p;  // [wave][head][D]
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) so[(w * G + h) * D + cl * EPL + e] = o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_wm[w][h] = m[h];
      s_wl[w][h] = l[h];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int h = e / D, dd = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < NW; ++x) M = fmaxf(M, s_wm[x][h]);
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const float mw = s_wm[x][h];
      const float al = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      O = fmaf(al, so[(x * G + h) * D + dd], O);
      L = fmaf(al, s_wl[x][h], L);
    }
    float *part = a.partials + ((head0 + h) * a.S + split) * (D + 2);
    if (dd == 0) {
      publish(part + 0, M);
      publish(part + 1, L);
    }
    publish(part + 2 + dd, O);
  }

  // ---- the last workgroup of this (b, g) merges all splits
  finish_split<D, G, NT, !FUSED>(a, head0, bg, split, &s_last, s_M, s_L, -1);
}

// ------------------------------------------------------------------ short contexts
// With few tokens (a compact H2O cache of 1280 slots, a prompt's first steps) the split-T layout
// above gives one workgroup per KV group, whose wavefronts each walk the whole union U of K'
// rows one batch after another: latency, not bandwidth.  Here a workgroup takes 256 tokens and
// its 4 wavefronts split the stored dims (wavefront w reads dims w, w + 4, ..., a dim that no
// head selected weighing 0).  Every K' and V load of the workgroup is issued first, so that the
// reads of the masks and q' (in the H2O form: the eviction and the selection) overlap them; the
// partial scores are added in LDS, then the tokens are split (64 per wavefront) for the softmax
// and the V pass.
// Partials, the last-workgroup merge and the mass update are as above.
//
// H2O form (the fused H2O step: one launch per decode step over a compact H2O cache whose every
// slot holds a token): eviction, the new token's K' and V, the group's selection and the
// mass-mode attention.  Each workgroup picks the victim itself (h2o_pick_victim on the masses as
// they stand: only the group's last workgroup writes them, after every other one has read them)
// and projects and selects the group's queries (fused_project_select).  The workgroup whose chunk
// holds the victim slot also projects the new key, and inside its chunk the slot's cached K' and
// V are replaced by the new token's (from LDS) in the partial scores and the V pass, so every
// number is the one the separate calls (aqua_h2o_victim, aqua_project_keys with slots,
// aqua_select_dims, aqua_decode in mass mode) compute.  That workgroup writes the new K' and V
// into the slot after its own reads of it; the group's last workgroup merges, sets the slot's
// position and restarts its mass from 0 before adding this step's weights.

// plain: aqua_decode.  step: aqua_decode_step at a short length, the H2O form's prologue with
// the new token going to column len - 1 (in place of a victim) and no slot bookkeeping.

template <typename KT, int D, int G, int MODE>
__device__ __forceinline__ void short_attend(const DecodeArgs &a, const H2OArgs &hh) {
  constexpr bool FUSED = MODE != kShortPlain;
  constexpr bool H2O = MODE == kShortH2O;
  constexpr int NT = 256;
  constexpr int NWORD = D / 32;
  constexpr int TPL = 4;                  // tokens per lane per K' row load
  constexpr int EPL = 16 / sizeof(KT);    // V elements per lane per 16-byte load
  constexpr int LPT = D / EPL;            // lanes per V row
  static_assert(LPT >= 8, "the V rows' lane butterfly starts at lane ^ 8");
  constexpr int TPI = 64 / LPT;           // V rows per wavefront load
  constexpr int RW = D / 4;               // most K' rows a wavefront reads
  constexpr int NL = 64 / TPI;            // V loads per lane
  typedef typename std::conditional<sizeof(KT) == 2, uint2, uint4>::type kvec;
  constexpr bool VPRO = FUSED && sizeof(KT) == 4;  // fp32 storage: projection on the VALU
  __shared__ __align__(16) float sP[VPRO ? D * D : 1];
  __shared__ __align__(16) float sq[VPRO ? G + 1 : 1][D];
  __shared__ float s_qp[FUSED ? G + 1 : 1][D];
  __shared__ uint32_t s_mw[FUSED ? G : 1][NWORD];
  __shared__ float s_knew[FUSED ? D : 1], s_vnew[FUSED ? D : 1];
  __shared__ float s_qw[D][G];                 // head weights of every stored dim (0: unselected)
  __shared__ float s_part[4][kShortChunk][G];  // partial scores; then the probabilities
  __shared__ float s_o[4][G][D];
  __shared__ float s_wm[4][G], s_wl[4][G], s_M[G], s_L[G];
  __shared__ int s_last;

  // every kernel argument read in one batch, and a grid of (chunk, KV head, batch): as in
  // decode_kernel
  asm volatile("" ::"s"(a.kp), "s"(a.v), "s"(a.q_proj), "s"(a.mask), "s"(a.q_raw), "s"(a.k_new),
               "s"(a.P), "s"(a.partials), "s"(a.mass), "s"(a.Hq), "s"(a.Hkv), "s"(a.d_store),
               "s"(a.T_cap), "s"(a.len), "s"(a.S), "s"(a.qscale), "s"(a.d_sel), "s"(a.k));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * a.Hkv + g;
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(g) * G;
  const size_t slot0 = static_cast<size_t>(bg) * a.T_cap;
  const int t0 = split * kShortChunk;
  if (!FUSED && tid == 0) install_epoch(&a.counters[bg], a.epoch);

  // ---- K' of this chunk, wavefront w's stored dims, every load in flight at once
  const int tl = min(t0 + TPL * lane, a.T_cap - TPL);  // stays inside the row; masked below
  const KT *kbase =
      static_cast<const KT *>(a.kp) + static_cast<size_t>(bg) * a.d_store * a.T_cap + tl;
  const int nw = a.d_store > w ? (a.d_store - w + 3) / 4 : 0;  // rows of this wavefront
  kvec kr[RW];
  auto load_k = [&]() {
#pragma unroll
    for (int i = 0; i < RW; ++i) {  // rows past nw re-read a stored row (never used)
      const int dim = i < nw ? w + 4 * i : min(w, a.d_store - 1);
      kr[i] = *reinterpret_cast<const kvec *>(kbase + static_cast<size_t>(dim) * a.T_cap);
    }
  };

  // ---- V of the wavefront's 64 tokens (t0 + 64 w ..).  K' and V loads go out here, or in the
  // fused forms once the prologue's own loads are on their way (held across those, their registers
  // would make the compiler issue P's loads one at a time)
  const int sub = lane / LPT, cl = lane - sub * LPT;
  const int last = a.len - 1;
  const KT *vbase = static_cast<const KT *>(a.v) + slot0 * D + cl * EPL;
  uint4 vr[NL];
  auto load_v = [&]() {
#pragma unroll
    for (int i = 0; i < NL; ++i) {  // rows past the last token re-read it (their p is 0)
      const int t = min(t0 + 64 * w + i * TPI + sub, last);
      vr[i] = load16(vbase + static_cast<size_t>(t) * D);
    }
  };
  if constexpr (!FUSED) {
    load_k();
    load_v();
  }

  int victim = -1;  // the column the new token goes to
  if constexpr (FUSED && !H2O) victim = a.len - 1;
  // H2O: the slots' masses and positions are requested here, and ranked only after the
  // prologue, so their round trip overlaps the prologue's; every workgroup keeps the new token's
  // K' and V in LDS meanwhile (the key is projected in every workgroup anyway; the victim's
  // owner uses them).  The compact cache fits one batch of the scan.
  static_assert(kDecodeShortMax <= 256 * kVictimBatch, "one batch of the victim scan");
  H2OVictimBatch vb;
  if constexpr (H2O) h2o_victim_load(a.mass + slot0, hh.slot_pos + slot0, a.len, tid, vb);
  const bool keep_new = H2O || (FUSED && victim >= t0 && victim < t0 + kShortChunk);
  if constexpr (FUSED) {
    auto issue = [&] {
      load_k();
      load_v();
    };
    if constexpr (sizeof(KT) == 2)  // K' at the start, V after the projection (see decode_kernel)
      fused_project_select_mfma<D, G, NT, true>(a, head0, bg, keep_new, split == 0, s_qp, s_mw,
                                                s_knew, s_vnew, load_k, load_v);
    else
      fused_project_select<KT, D, G, NT>(a, head0, bg, keep_new, split == 0, sP, sq, s_qp, s_mw,
                                         s_knew, s_vnew, issue);
  }
  if constexpr (H2O) {
    uint64_t key = ~0ull;
    int slot = 0x7fffffff;
    h2o_victim_fold(vb, a.len, tid, hh.t_new - hh.recent, key, slot);
    victim = h2o_victim_reduce(key, slot);
    if (split == 0 && tid == 0) hh.victim[bg] = victim;
  }
  const bool owner = FUSED && victim >= t0 && victim < t0 + kShortChunk;  // false if victim is -1

  // ---- every stored dim's weight per head: q'_i * scale * log2 e where the head selected it
  if (tid < a.d_store) {
    const int wd = tid >> 5, bit = tid & 31;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint32_t mw;
      float qv;
      if constexpr (FUSED) {
        mw = s_mw[h][wd];
        qv = s_qp[h][tid];
      } else {
        mw = a.mask[(head0 + h) * NWORD + wd];
        qv = a.q_proj[(head0 + h) * D + tid];
      }
      s_qw[tid][h] = ((mw >> bit) & 1u) ? qv * a.qscale : 0.0f;
    }
  }
  __syncthreads();

  // ---- partial scores (the victim slot, in the owner's chunk, takes the new token's K')
  const int vj = owner ? victim - tl : -1;  // the victim's token among this lane's four
  float acc[G][TPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < TPL; ++j) acc[h][j] = 0.0f;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if (i < nw) {  // uniform over the wavefront
      float kv[TPL];
      if constexpr (sizeof(KT) == 2) {
        kv[0] = bf16_lo(kr[i].x); kv[1] = bf16_hi(kr[i].x);
        kv[2] = bf16_lo(kr[i].y); kv[3] = bf16_hi(kr[i].y);
      } else {
        kv[0] = __uint_as_float(kr[i].x); kv[1] = __uint_as_float(kr[i].y);
        kv[2] = __uint_as_float(kr[i].z); kv[3] = __uint_as_float(kr[i].w);
      }
      const int dim = w + 4 * i;
      if constexpr (FUSED) {
#pragma unroll
        for (int j = 0; j < TPL; ++j)
          if (j == vj) kv[j] = s_knew[dim];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float qw = s_qw[dim][h];
#pragma unroll
        for (int j = 0; j < TPL; ++j) acc[h][j] = fmaf(qw, kv[j], acc[h][j]);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < TPL; ++j)
#pragma unroll
    for (int h = 0; h < G; ++h) s_part[w][TPL * lane + j][h] = acc[h][j];
  __syncthreads();

  // ---- wavefront w now owns tokens t0 + 64 w + lane: full scores, softmax numerators
  const int lt = 64 * w + lane, tk = t0 + lt;
  const bool valid = tk < a.len;
  float sc[G], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = s_part[0][lt][h] + s_part[1][lt][h] + s_part[2][lt][h] + s_part[3][lt][h];
    sc[h] = valid ? x : -INFINITY;
    if (a.mass && valid) publish(a.scores + (head0 + h) * a.T_cap + tk, sc[h]);
    m[h] = wave_max(sc[h]);
    const float p = (m[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[h] - m[h]);
    l[h] = wave_sum(p);
    s_part[0][lt][h] = p;  // only this wavefront reads its own tokens' slots
  }

  // ---- o = sum_t p_t V_t over the wavefront's 64 tokens (the victim slot: the new V)
  float o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    float vv[EPL];
    Vec<KT>::unpack(vr[i], vv);
    if constexpr (FUSED) {
      if (owner && min(t0 + 64 * w + i * TPI + sub, last) == victim) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = s_vnew[cl * EPL + e];
      }
    }
    const int r = 64 * w + i * TPI + sub;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = s_part[0][r][h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p, vv[e], o[h][e]);
    }
  }
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = add_xor(o[h][e], off);

  // ---- merge the 4 wavefronts, write this chunk's partials
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[w][h][cl * EPL + e] = o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_wm[w][h] = m[h];
      s_wl[w][h] = l[h];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int h = e / D, dd = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < 4; ++x) M = fmaxf(M, s_wm[x][h]);
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float mw = s_wm[x][h];
      const float al = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      O = fmaf(al, s_o[x][h][dd], O);
      L = fmaf(al, s_wl[x][h], L);
    }
    float *part = a.partials + ((head0 + h) * a.S + split) * (D + 2);
    if (dd == 0) {
      publish(part + 0, M);
      publish(part + 1, L);
    }
    publish(part + 2 + dd, O);
  }
  if constexpr (FUSED) {
    // the new token into the victim slot: this workgroup's reads of the slot are consumed
    if (owner && tid < D) {
      if (tid < a.d_store)
        static_cast<KT *>(a.kp_w)[(static_cast<size_t>(bg) * a.d_store + tid) * a.T_cap +
                                  victim] = store_elem<KT>(s_knew[tid]);
      static_cast<KT *>(a.v_w)[(slot0 + victim) * D + tid] = store_elem<KT>(s_vnew[tid]);
    }
  }

  // ---- the last workgroup of this (b, g) merges all chunks (and updates the masses); a short
  // context has at most 16 chunks, one merge level
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partials, scores and cache writes have landed
  __syncthreads();
  if (tid == 0)
    s_last = arrive_last(&a.counters[bg], a.epoch, static_cast<uint32_t>(a.S), !FUSED);
  __syncthreads();
  if (!s_last) return;
  if (H2O && victim >= 0 && tid == 0) hh.slot_pos[slot0 + victim] = hh.t_new;
  merge_splits<D, G, NT>(a, head0, bg, s_M, s_L, H2O ? victim : -1, a.S, 1);
}

template <typename KT, int D, int G>
__global__ __launch_bounds__(256) void decode_short_kernel(DecodeArgs a) {
  short_attend<KT, D, G, kShortPlain>(a, H2OArgs{});
}

// The fused forms let each wavefront take a whole SIMD's registers: its K' and V loads, P's parts
// (or, for fp32 storage, P staged in LDS) and the victim's then all stay in flight together.
template <typename KT, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_step_short_kernel(DecodeArgs a) {
  short_attend<KT, D, G, kShortStep>(a, H2OArgs{});
}

template <typename KT, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void h2o_step_kernel(DecodeArgs a, H2OArgs hh) {
  short_attend<KT, D, G, kShortH2O>(a, hh);
}


// ------------------------------------------------------------------ launch helpers
// (each translation unit that includes this header instantiates the forms it launches)
template <typename KT, int D, int G, bool FUSED>
hipError_t launch_split_g(const DecodeArgs &a, const DecodeLayout &L, hipStream_t s) {
  if (a.S != (a.len + L.split - 1) / L.split) return hipErrorInvalidConfiguration;
  const dim3 grid(a.S, a.Hkv, a.B);
  if constexpr (G == 4 || G == 8) {
    if (L.waves == 8) {
      decode_kernel<KT, D, G, 8, FUSED><<<grid, dim3(512), 0, s>>>(a);
      return hipGetLastError();
    }
  }
  constexpr int NW = 4;
  if (L.waves != NW) return hipErrorInvalidConfiguration;
  decode_kernel<KT, D, G, NW, FUSED><<<grid, dim3(NW * 64), 0, s>>>(a);
  return hipGetLastError();
}

template <typename KT, int D, bool FUSED>
hipError_t launch_split_d(const DecodeArgs &a, const DecodeLayout &L, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_split_g<KT, D, 1, FUSED>(a, L, s);
    case 2: return launch_split_g<KT, D, 2, FUSED>(a, L, s);
    case 4: return launch_split_g<KT, D, 4, FUSED>(a, L, s);
    default: return launch_split_g<KT, D, 8, FUSED>(a, L, s);
  }
}

template <typename KT, bool FUSED>
hipError_t launch_split_t(const DecodeArgs &a, const DecodeLayout &L, hipStream_t s) {
  return a.d == 128 ? launch_split_d<KT, 128, FUSED>(a, L, s)
                    : launch_split_d<KT, 64, FUSED>(a, L, s);
}

template <typename KT, int D, int G, int MODE>
hipError_t launch_short_g(const DecodeArgs &a, const H2OArgs &h, hipStream_t s) {
  if (a.S != (a.len + kShortChunk - 1) / kShortChunk) return hipErrorInvalidConfiguration;
  const dim3 grid(a.S, a.Hkv, a.B), block(256);
  if constexpr (MODE == kShortH2O) h2o_step_kernel<KT, D, G><<<grid, block, 0, s>>>(a, h);
  else if constexpr (MODE == kShortStep) decode_step_short_kernel<KT, D, G><<<grid, block, 0, s>>>(a);
  else decode_short_kernel<KT, D, G><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <typename KT, int D, int MODE>
hipError_t launch_short_d(const DecodeArgs &a, const H2OArgs &h, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_short_g<KT, D, 1, MODE>(a, h, s);
    case 2: return launch_short_g<KT, D, 2, MODE>(a, h, s);
    case 4: return launch_short_g<KT, D, 4, MODE>(a, h, s);
    default: return launch_short_g<KT, D, 8, MODE>(a, h, s);
  }
}

template <typename KT, int MODE>
hipError_t launch_short_t(const DecodeArgs &a, const H2OArgs &h, hipStream_t s) {
  return a.d == 128 ? launch_short_d<KT, 128, MODE>(a, h, s)
                    : launch_short_d<KT, 64, MODE>(a, h, s);
}

}  // namespace
}  // namespace aqua
