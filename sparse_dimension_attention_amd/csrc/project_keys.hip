// Online key projection into the dimension-major K' cache (AQUA's online step projects keys with
// the offline matrix: digest of arXiv 2509.11155, section 方法详解 / 技术框架; edgentiq blog, "How
// AQUA Works", step 2).  Only dims 0..d_store-1 are kept (AQUA-Memory's static cut, blog section
// "AQUA-Memory").  V is copied unchanged.
//
// One workgroup per tile of TT tokens of one (b, g).  The raw keys are staged in LDS as fp32;
// thread (i, group) computes K'[t][i] = sum_j K[t][j] P[j][i] for its tokens (j ascending, fma),
// reading P's row j coalesced across i and K[t][j..j+3] as an LDS broadcast.  The results are
// rounded once to the storage type and transposed through LDS, so that each wavefront then
// writes 64 consecutive token columns of one K' row.
#include "aqua_internal.h"

namespace aqua {
namespace {

template <typename KT, int D>
struct ProjCfg {
  static constexpr int TT = sizeof(KT) == 2 ? 64 : 32;  // tokens per workgroup (LDS <= 64 KB)
  static constexpr int TG = 256 / D;                    // token groups per workgroup
  static constexpr int TPT = TT / TG;                   // tokens per thread
};

template <typename KT, int D>
__global__ __launch_bounds__(256) void project_keys_kernel(
    const KT *__restrict__ k_raw, const KT *__restrict__ v_raw, const float *__restrict__ P,
    int n, int d_store, int T_cap, int len0, const int32_t *__restrict__ slots,
    KT *__restrict__ kp, KT *__restrict__ vc) {
  using C = ProjCfg<KT, D>;
  constexpr int TT = C::TT, TPT = C::TPT;
  __shared__ float ks[TT][D + 4];
  __shared__ KT kt[D][TT + 2];
  __shared__ int cols[TT];

  const int bg = blockIdx.y;
  const int t0 = blockIdx.x * TT;
  const int nt = min(TT, n - t0);
  const int tid = threadIdx.x;

  for (int e = tid; e < TT * D; e += 256) {
    const int t = e / D, j = e % D;
    ks[t][j] = (t < nt) ? load_elem<KT>(k_raw + (static_cast<size_t>(bg) * n + t0 + t) * D + j)
                        : 0.0f;
  }
  if (tid < TT) {
    int col = -1;
    if (tid < nt) col = slots ? slots[static_cast<size_t>(bg) * n + t0 + tid] : len0 + t0 + tid;
    cols[tid] = (col >= 0 && col < T_cap) ? col : -1;
  }
  __syncthreads();

  const int i = tid % D, tg = tid / D;
  float acc[TPT];
#pragma unroll
  for (int r = 0; r < TPT; ++r) acc[r] = 0.0f;
  for (int j = 0; j < D; j += 4) {
    const float p0 = P[(j + 0) * D + i], p1 = P[(j + 1) * D + i];
    const float p2 = P[(j + 2) * D + i], p3 = P[(j + 3) * D + i];
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const float4 kv = *reinterpret_cast<const float4 *>(&ks[tg * TPT + r][j]);
      float a = acc[r];
      a = fmaf(kv.x, p0, a);
      a = fmaf(kv.y, p1, a);
      a = fmaf(kv.z, p2, a);
      a = fmaf(kv.w, p3, a);
      acc[r] = a;
    }
  }
#pragma unroll
  for (int r = 0; r < TPT; ++r) kt[i][tg * TPT + r] = store_elem<KT>(acc[r]);
  __syncthreads();

  // K' rows: each wavefront writes consecutive token columns of one dimension row.
  for (int e = tid; e < d_store * TT; e += 256) {
    const int row = e / TT, t = e % TT;
    const int col = cols[t];
    if (t < nt && col >= 0)
      kp[(static_cast<size_t>(bg) * d_store + row) * T_cap + col] = kt[row][t];
  }
  // V rows, 16 bytes per thread
  if (v_raw) {
    constexpr int VEC = 16 / sizeof(KT);
    constexpr int PER_ROW = D / VEC;
    for (int e = tid; e < nt * PER_ROW; e += 256) {
      const int t = e / PER_ROW, c = e % PER_ROW;
      const int col = cols[t];
      if (col < 0) continue;
      const uint4 val = *reinterpret_cast<const uint4 *>(
          v_raw + (static_cast<size_t>(bg) * n + t0 + t) * D + c * VEC);
      *reinterpret_cast<uint4 *>(vc + (static_cast<size_t>(bg) * T_cap + col) * D + c * VEC) =
          val;
    }
  }
}

// Few tokens per (b, g), as in a decode step: one workgroup of 256 threads per (b, g) stages
// P in LDS with 16-byte loads (all in flight at once: one L2 round trip), then thread i < D
// owns projected dimension i of every token (P's row j read from LDS, consecutive banks).
constexpr int kSmallN = 8;

template <typename KT, int D>
__global__ __launch_bounds__(256) void project_keys_small_kernel(
    const KT *__restrict__ k_raw, const KT *__restrict__ v_raw, const float *__restrict__ P,
    int n, int d_store, int T_cap, int len0, const int32_t *__restrict__ slots,
    KT *__restrict__ kp, KT *__restrict__ vc) {
  __shared__ float sP[D * D];
  __shared__ float ks[kSmallN][D];
  __shared__ int cols[kSmallN];
  const int bg = blockIdx.x, tid = threadIdx.x;
  {
    constexpr int NV = D * D / (256 * 4);
    float4 st[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
      st[v] = *reinterpret_cast<const float4 *>(&P[(v * 256 + tid) * 4]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < NV; ++v) *reinterpret_cast<float4 *>(&sP[(v * 256 + tid) * 4]) = st[v];
  }
  for (int e = tid; e < n * D; e += 256)
    ks[e / D][e % D] = load_elem<KT>(k_raw + static_cast<size_t>(bg) * n * D + e);
  if (tid < n) {
    const int col = slots ? slots[static_cast<size_t>(bg) * n + tid] : len0 + tid;
    cols[tid] = (col >= 0 && col < T_cap) ? col : -1;
  }
  __syncthreads();
  if (tid < D) {
    // one fully unrolled, branch-free j chain per token: the LDS reads are issued ahead
    const int i = tid;
    for (int t = 0; t < n; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < D; ++j) acc = fmaf(ks[t][j], sP[j * D + i], acc);
      if (i < d_store && cols[t] >= 0)
        kp[(static_cast<size_t>(bg) * d_store + i) * T_cap + cols[t]] = store_elem<KT>(acc);
    }
  }
  if (v_raw) {
    for (int e = tid; e < n * D; e += 256) {
      const int t = e / D;
      if (cols[t] >= 0)
        vc[(static_cast<size_t>(bg) * T_cap + cols[t]) * D + e % D] =
            v_raw[static_cast<size_t>(bg) * n * D + e];
    }
  }
}

template <typename KT, int D>
hipError_t launch_pk(const void *k_raw, const void *v_raw, const float *P, int B, int Hkv, int n,
                     int d_store, int T_cap, int len0, const int32_t *slots, void *kp, void *v,
                     hipStream_t s) {
  using C = ProjCfg<KT, D>;
  if (n <= kSmallN) {
    project_keys_small_kernel<KT, D><<<dim3(B * Hkv), dim3(256), 0, s>>>(
        static_cast<const KT *>(k_raw), static_cast<const KT *>(v_raw), P, n, d_store, T_cap,
        len0, slots, static_cast<KT *>(kp), static_cast<KT *>(v));
    return hipGetLastError();
  }
  const dim3 grid((n + C::TT - 1) / C::TT, B * Hkv), block(256);
  project_keys_kernel<KT, D><<<grid, block, 0, s>>>(
      static_cast<const KT *>(k_raw), static_cast<const KT *>(v_raw), P, n, d_store, T_cap, len0,
      slots, static_cast<KT *>(kp), static_cast<KT *>(v));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project_keys(int dtype, const void *k_raw, const void *v_raw, const float *P,
                               int B, int Hkv, int n, int d, int d_store, int T_cap, int len0,
                               const int32_t *slots, void *kp, void *v, hipStream_t s) {
  if (dtype == 1)
    return d == 128 ? launch_pk<bf16_t, 128>(k_raw, v_raw, P, B, Hkv, n, d_store, T_cap, len0,
                                             slots, kp, v, s)
                    : launch_pk<bf16_t, 64>(k_raw, v_raw, P, B, Hkv, n, d_store, T_cap, len0,
                                            slots, kp, v, s);
  return d == 128 ? launch_pk<float, 128>(k_raw, v_raw, P, B, Hkv, n, d_store, T_cap, len0,
                                          slots, kp, v, s)
                  : launch_pk<float, 64>(k_raw, v_raw, P, B, Hkv, n, d_store, T_cap, len0, slots,
                                         kp, v, s);
}

}  // namespace aqua
