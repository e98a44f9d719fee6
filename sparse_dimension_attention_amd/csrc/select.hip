// Query projection and per-query top-k dimension selection (AQUA's dynamic selection by
// projected-query magnitude: digest of arXiv 2509.11155, section 方法详解 / 核心思路 and 技术框架;
// edgentiq blog, "How AQUA Works", step 2).
//
// Projection: q'_i = sum_j q_j P[j][i] at fp32 accuracy.  bf16 queries take the library's one
// bf16 projection (proj_mfma: v_mfma_f32_16x16x32_bf16 on P's exact three-part bf16 split), the
// arithmetic the fused decode and H2O steps and the prefill use too; fp32 queries take an fma
// chain over j ascending on the VALU, with P staged in LDS.
//
// Selection, one wavefront per row: lane l owns projected dims l and l + 64 (d = 128) or dim l
// (d = 64), so that the 64-bit ballot of "dim selected" over the lanes is directly the mask word
// pair of dims 0..63 (and 64..127); wave_topk_threshold compares sign-cleared fp32 bit patterns
// exactly, ties to the lower index, building the k-th largest key MSB first from wave ballots and
// stopping as soon as exactly k keys clear the running threshold.
#include "aqua_internal.h"

namespace aqua {
namespace {

// The outputs of one selected row: q' (if asked for), the mask words (lane l < D/32 writes word
// l: bits of dims 32 l .. 32 l + 31) and the ascending index list (if asked for).
template <int D>
__device__ __forceinline__ void write_selection(int row, const float (&x)[D / 64],
                                                const bool (&sel)[D / 64], int k,
                                                float *__restrict__ q_proj,
                                                uint32_t *__restrict__ mask,
                                                int16_t *__restrict__ idx) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  uint64_t sb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sb[e] = __ballot(sel[e]);
  if (q_proj) {
#pragma unroll
    for (int e = 0; e < E; ++e) q_proj[static_cast<size_t>(row) * D + lane + 64 * e] = x[e];
  }
  if (lane < D / 32) {
    const uint64_t b = (lane >> 1) ? sb[E - 1] : sb[0];
    mask[static_cast<size_t>(row) * (D / 32) + lane] =
        (lane & 1) ? static_cast<uint32_t>(b >> 32) : static_cast<uint32_t>(b);
  }
  if (idx) {
    int before = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int pos = before + __builtin_amdgcn_mbcnt_hi(
                                   static_cast<uint32_t>(sb[e] >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(sb[e]), 0u));
      if (sel[e]) idx[static_cast<size_t>(row) * k + pos] = static_cast<int16_t>(lane + 64 * e);
      before += __popcll(sb[e]);
    }
  }
}

// fp32 queries (VALU): P staged in LDS, one wavefront per row.
template <int D>
__global__ __launch_bounds__(256) void select_kernel(const float *__restrict__ q, int N,
                                                     const float *__restrict__ P, int d_sel,
                                                     int k, float *__restrict__ q_proj,
                                                     uint32_t *__restrict__ mask,
                                                     int16_t *__restrict__ idx) {
  constexpr int E = D / 64;  // dims per lane: lane, lane + 64
  __shared__ float sP[D * D];
  {
    constexpr int NV = D * D / (256 * 4);  // float4 per thread; all in flight at once
    float4 st[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
      st[v] = *reinterpret_cast<const float4 *>(&P[(v * 256 + threadIdx.x) * 4]);
    __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first LDS store
#pragma unroll
    for (int v = 0; v < NV; ++v) *reinterpret_cast<float4 *>(&sP[(v * 256 + threadIdx.x) * 4]) = st[v];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;  // whole wave leaves; no workgroup barrier follows

  const float *qr = q + static_cast<size_t>(row) * D;
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = qr[lane + 64 * e];

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const float src = (j < 64) ? qv[0] : qv[E - 1];
    const float qj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), j & 63));
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(qj, sP[j * D + lane + 64 * e], acc[e]);
  }

  bool sel[E];
  wave_topk_threshold<E>(acc, d_sel, k, sel);
  write_selection<D>(row, acc, sel, k, q_proj, mask, idx);
}

// bf16 queries (MFMA): a workgroup of D/16 wavefronts takes 16 rows; wavefront w projects output
// columns [16 w, 16 w + 16) with proj_mfma (the library's one bf16 projection), the q' tile goes
// through LDS, and each wavefront then selects 16 / (D/16) of the rows.
template <int D>
__global__ __launch_bounds__(D / 16 * 64) void select_mfma_kernel(
    const bf16_t *__restrict__ q, int N, const float *__restrict__ P, int d_sel, int k,
    float *__restrict__ q_proj, uint32_t *__restrict__ mask, int16_t *__restrict__ idx) {
  constexpr int KS = D / 32, NB = D / 16, RPW = 16 / NB, E = D / 64;
  __shared__ float tile[16][D + 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 16;
  u32x4_t av[KS];
  load_a_row<KS>(q + static_cast<size_t>(min(r0 + (lane & 15), N - 1)) * D, av);
  PParts<KS> pp;
  load_p_parts<KS>(P, 16 * w, pp);
  const f32x4_t x = proj_mfma<KS>(av, pp);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) tile[4 * (lane >> 4) + rr][16 * w + (lane & 15)] = x[rr];
  __syncthreads();
  for (int i = 0; i < RPW; ++i) {
    const int rl = w * RPW + i, row = r0 + rl;
    if (row >= N) break;  // uniform over the wavefront; no barrier follows
    float xs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) xs[e] = tile[rl][lane + 64 * e];
    bool sel[E];
    wave_topk_threshold<E>(xs, d_sel, k, sel);
    write_selection<D>(row, xs, sel, k, q_proj, mask, idx);
  }
}

}  // namespace

hipError_t launch_select(const void *q, int qdt, int N, int d, const float *P, int d_sel, int k,
                         float *q_proj, uint32_t *mask, int16_t *idx, hipStream_t s) {
  if (qdt == 0) {
    const dim3 grid((N + 3) / 4), block(256);
    if (d == 128)
      select_kernel<128><<<grid, block, 0, s>>>(static_cast<const float *>(q), N, P, d_sel, k,
                                                q_proj, mask, idx);
    else
      select_kernel<64><<<grid, block, 0, s>>>(static_cast<const float *>(q), N, P, d_sel, k,
                                               q_proj, mask, idx);
  } else {
    const dim3 grid((N + 15) / 16);
    if (d == 128)
      select_mfma_kernel<128><<<grid, dim3(512), 0, s>>>(static_cast<const bf16_t *>(q), N, P,
                                                         d_sel, k, q_proj, mask, idx);
    else
      select_mfma_kernel<64><<<grid, dim3(256), 0, s>>>(static_cast<const bf16_t *>(q), N, P,
                                                        d_sel, k, q_proj, mask, idx);
  }
  return hipGetLastError();
}

}  // namespace aqua
