// GQA decode attention over each query's selected projected dimensions (AQUA: attention
// computed on the dims kept by projected-query magnitude; digest of arXiv 2509.11155, section
// 方法详解 / 技术框架; edgentiq blog, "How AQUA Works", step 2), split over the context with a
// final flash-decoding style combination of (max, sum, weighted V) partials.
//
// Memory-bound design for one (b, KV group g) and one split of the context per workgroup:
//  * The G query heads of a KV group each keep their own dims; the workgroup reads the K' rows
//    of the union U of those masks, once, and every head uses its own masked q' (zero on dims it
//    did not keep).  K' is dimension-major, so each selected row is a contiguous run of tokens:
//    lane l reads 16 bytes (8 bf16 / 4 fp32 tokens) of a row, a wavefront 1 KiB, fully coalesced;
//    rows outside U are never touched.
//  * Each wavefront owns a contiguous run of 64 * 16/sizeof(elem) tokens and computes all of
//    its scores before any exponential, so there is no running rescale inside a wavefront.
//    Scores live in log2 units (q' pre-multiplied by scale * log2 e) and use v_exp_f32.
//  * The softmax numerators go through LDS to the V pass, where 16 bytes per lane cover a V
//    row (d = 128 bf16: 16 lanes per token, 4 tokens per wavefront load).
//  * The workgroup's wavefronts merge their (m, l, o) in LDS; the workgroup writes one partial
//    per query head.  The last workgroup of a (b, g) to finish (atomic counter in the
//    workspace) merges all partials of the group, writes the output and resets its counter.
//  * H2O mass mode additionally stores the raw scores and lets that last workgroup add every
//    token's normalised probability, summed over the group's heads, to its mass.
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
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename KT, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  constexpr int TPL = Vec<KT>::N;  // tokens per lane per K' row load
  constexpr int WT = 64 * TPL;     // tokens per wavefront
  constexpr int EPL = Vec<KT>::N;  // V elements per lane per load
  constexpr int LPT = D / EPL;     // lanes per V row
  constexpr int TPI = 64 / LPT;    // V rows per wavefront load
  constexpr int NWORD = D / 32;
  constexpr int NT = NW * 64;
  static_assert(WT % (TPI * kUnroll) == 0, "V loop tiling");
  static_assert(NW * G * D <= NW * WT * G, "LDS reuse");

  __shared__ int s_dl[D];
  __shared__ float s_qw[D][G];
  __shared__ float s_p[NW * WT * G];  // [wave][token][head]; reused for the wave merge
  __shared__ float s_wm[NW][G], s_wl[NW][G];
  __shared__ float s_M[G], s_L[G];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bg = blockIdx.x / a.S, split = blockIdx.x - bg * a.S;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(g) * G;

  // ---- union of the group's masks, restricted to stored dims (uniform per workgroup)
  uint32_t U[NWORD];
  int nU = 0, last_dim = 0;
#pragma unroll
  for (int wd = 0; wd < NWORD; ++wd) {
    uint32_t u = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) u |= a.mask[(head0 + h) * NWORD + wd];
    const int lo = wd * 32;
    if (a.d_store <= lo) u = 0;
    else if (a.d_store < lo + 32) u &= (1u << (a.d_store - lo)) - 1u;
    U[wd] = u;
    nU += __popc(u);
    if (u) last_dim = lo + 31 - __clz(u);
  }
  // padded to whole batches with the last dim at zero weight (re-reads hit in cache)
  const int nUp = (nU + kUnroll - 1) / kUnroll * kUnroll;
  if (tid < D) {
    const int wd = tid >> 5, bit = tid & 31;
    uint32_t mw[G];
    float qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mw[h] = a.mask[(head0 + h) * NWORD + wd];
      qv[h] = a.q_proj[(head0 + h) * D + tid];
    }
    uint32_t uw = 0;
    int pos = 0;
#pragma unroll
    for (int x = 0; x < NWORD; ++x) {
      if (x < wd) pos += __popc(U[x]);
      if (x == wd) uw = U[x];
    }
    if ((uw >> bit) & 1u) {
      pos += __popc(uw & ((1u << bit) - 1u));
      s_dl[pos] = tid;
#pragma unroll
      for (int h = 0; h < G; ++h) s_qw[pos][h] = ((mw[h] >> bit) & 1u) ? qv[h] * a.qscale : 0.0f;
    }
    if (tid >= nU && tid < nUp) {
      s_dl[tid] = last_dim;
#pragma unroll
      for (int h = 0; h < G; ++h) s_qw[tid][h] = 0.0f;
    }
  }
  __syncthreads();

  // ---- phase 1: log2-domain scores of this wavefront's tokens
  // Lanes past len read the last valid 16-byte chunk instead (same cache line as a live lane);
  // their scores are discarded below.  Loads are unconditional so that the prefetch of the
  // next batch overlaps the arithmetic of the current one (vmcnt stays at one batch).
  const int tw0 = split * (NW * WT) + w * WT;
  const int tl = tw0 + lane * TPL;
  const bool wave_live = tw0 < a.len;
  const int tl_ld = min(tl, ((a.len - 1) / TPL) * TPL);
  const KT *kbase = static_cast<const KT *>(a.kp) +
                    static_cast<size_t>(bg) * a.d_store * a.T_cap + tl_ld;
  float acc[G][TPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < TPL; ++j) acc[h][j] = 0.0f;

  auto k_load = [&](uint4 (&buf)[kUnroll], int u) {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      buf[i] = load16(kbase + static_cast<size_t>(s_dl[u + i]) * a.T_cap);
  };
  auto k_fma = [&](const uint4 (&buf)[kUnroll], int u) {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      float kv[TPL];
      Vec<KT>::unpack(buf[i], kv);
      float qw[G];
#pragma unroll
      for (int h = 0; h < G; ++h) qw[h] = s_qw[u + i][h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < TPL; ++j) acc[h][j] = fmaf(qw[h], kv[j], acc[h][j]);
    }
  };
  if (wave_live && nUp > 0) {
    uint4 bA[kUnroll], bB[kUnroll];
    k_load(bA, 0);
    for (int u = 0;;) {
      if (u + kUnroll >= nUp) { k_fma(bA, u); break; }
      k_load(bB, u + kUnroll);
      k_fma(bA, u);
      u += kUnroll;
      if (u + kUnroll >= nUp) { k_fma(bB, u); break; }
      k_load(bA, u + kUnroll);
      k_fma(bB, u);
      u += kUnroll;
    }
  }

  // ---- softmax numerators within the wavefront
#pragma unroll
  for (int j = 0; j < TPL; ++j)
    if (tl + j >= a.len)
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h][j] = -INFINITY;
  if (a.mass) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < TPL; ++j)
        if (tl + j < a.len) a.scores[(head0 + h) * a.T_cap + tl + j] = acc[h][j];
  }
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = acc[h][0];
#pragma unroll
    for (int j = 1; j < TPL; ++j) mx = fmaxf(mx, acc[h][j]);
    m[h] = wave_max(mx);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      const float p = (m[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(acc[h][j] - m[h]);
      acc[h][j] = p;
      sum += p;
    }
    l[h] = wave_sum(sum);
  }
  float *sp = s_p + w * (WT * G);
#pragma unroll
  for (int j = 0; j < TPL; ++j)
#pragma unroll
    for (int h = 0; h < G; ++h) sp[(lane * TPL + j) * G + h] = acc[h][j];
  __syncthreads();

  // ---- phase 2: o = sum_t p_t V_t over this wavefront's tokens
  // Rows past len read the last valid row (their p is 0), again to keep loads unconditional.
  const int sub = lane / LPT, cl = lane - sub * LPT;
  const int nrow = min(WT, a.len - tw0);  // may be <= 0
  const KT *vbase = static_cast<const KT *>(a.v) +
                    (static_cast<size_t>(bg) * a.T_cap + tw0) * D + cl * EPL;
  float o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
  constexpr int RB = TPI * kUnroll;  // rows per batch
  auto v_load = [&](uint4 (&buf)[kUnroll], int r0) {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int t = min(r0 + i * TPI + sub, nrow - 1);
      buf[i] = load16(vbase + static_cast<size_t>(t) * D);
    }
  };
  auto v_fma = [&](const uint4 (&buf)[kUnroll], int r0) {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int t = r0 + i * TPI + sub;
      float vv[EPL];
      Vec<KT>::unpack(buf[i], vv);
      float p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) p[h] = sp[t * G + h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p[h], vv[e], o[h][e]);
    }
  };
  if (nrow > 0) {
    uint4 bA[kUnroll], bB[kUnroll];
    v_load(bA, 0);
    for (int r0 = 0;;) {
      if (r0 + RB >= nrow) { v_fma(bA, r0); break; }
      v_load(bB, r0 + RB);
      v_fma(bA, r0);
      r0 += RB;
      if (r0 + RB >= nrow) { v_fma(bB, r0); break; }
      v_load(bA, r0 + RB);
      v_fma(bB, r0);
      r0 += RB;
    }
  }
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] += __shfl_xor(o[h][e], off, 64);
  __syncthreads();  // every wavefront is done with s_p

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
      part[0] = M;
      part[1] = L;
    }
    part[2 + dd] = O;
  }

  // ---- the last workgroup of this (b, g) merges all splits
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&a.counters[bg], 1u) == static_cast<unsigned>(a.S - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  for (int e = tid; e < G * D; e += NT) {
    const int h = e / D, dd = e - h * D;
    const float *part = a.partials + (head0 + h) * a.S * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.S; ++s) M = fmaxf(M, coherent_load(part + s * (D + 2)));
    float O = 0.0f, L = 0.0f;
    for (int s = 0; s < a.S; ++s) {
      const float ms = coherent_load(part + s * (D + 2));
      const float al = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
      L = fmaf(al, coherent_load(part + s * (D + 2) + 1), L);
      O = fmaf(al, coherent_load(part + s * (D + 2) + 2 + dd), O);
    }
    a.out[(head0 + h) * D + dd] = O / L;
    if (dd == 0) {
      s_M[h] = M;
      s_L[h] = L;
    }
  }
  if (a.mass) {
    __syncthreads();
    float *mass = a.mass + static_cast<size_t>(bg) * a.T_cap;
    for (int t = tid; t < a.len; t += NT) {
      float add = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h)
        add += __builtin_amdgcn_exp2f(coherent_load(a.scores + (head0 + h) * a.T_cap + t) -
                                      s_M[h]) / s_L[h];
      mass[t] += add;
    }
  }
  if (tid == 0) atomicExch(&a.counters[bg], 0u);
}

template <typename KT, int D, int G>
hipError_t launch_g(const DecodeArgs &a, hipStream_t s) {
  constexpr int NW = (G == 8) ? 2 : 4;
  const dim3 grid(a.B * a.Hkv * a.S), block(NW * 64);
  decode_kernel<KT, D, G, NW><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <typename KT, int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<KT, D, 1>(a, s);
    case 2: return launch_g<KT, D, 2>(a, s);
    case 4: return launch_g<KT, D, 4>(a, s);
    default: return launch_g<KT, D, 8>(a, s);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

DecodeLayout decode_layout(int dtype, int G) {
  DecodeLayout L;
  L.waves = (G == 8) ? 2 : 4;
  L.tokens_wave = 64 * (dtype == 1 ? 8 : 4);
  L.split = L.waves * L.tokens_wave;
  return L;
}

size_t decode_workspace_bytes(int dtype, int B, int Hq, int Hkv, int d, int T_cap) {
  const DecodeLayout L = decode_layout(dtype, Hq / Hkv);
  const size_t S = (static_cast<size_t>(T_cap) + L.split - 1) / L.split;
  return align256(static_cast<size_t>(B) * Hkv * 4) +
         align256(static_cast<size_t>(B) * Hq * S * (d + 2) * 4) +
         static_cast<size_t>(B) * Hq * T_cap * 4;
}

void decode_workspace_carve(void *ws, int dtype, int B, int Hq, int Hkv, int d, int T_cap,
                            uint32_t **counters, float **partials, float **scores) {
  const DecodeLayout L = decode_layout(dtype, Hq / Hkv);
  const size_t S = (static_cast<size_t>(T_cap) + L.split - 1) / L.split;
  char *p = static_cast<char *>(ws);
  *counters = reinterpret_cast<uint32_t *>(p);
  p += align256(static_cast<size_t>(B) * Hkv * 4);
  *partials = reinterpret_cast<float *>(p);
  p += align256(static_cast<size_t>(B) * Hq * S * (d + 2) * 4);
  *scores = reinterpret_cast<float *>(p);
}

hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s) {
  if (dtype == 1) return a.d == 128 ? launch_d<bf16_t, 128>(a, s) : launch_d<bf16_t, 64>(a, s);
  return a.d == 128 ? launch_d<float, 128>(a, s) : launch_d<float, 64>(a, s);
}

}  // namespace aqua
