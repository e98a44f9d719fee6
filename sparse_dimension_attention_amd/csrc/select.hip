// Query projection and per-query top-k dimension selection (AQUA's dynamic selection by
// projected-query magnitude: digest of arXiv 2509.11155, section 方法详解 / 核心思路 and 技术框架;
// edgentiq blog, "How AQUA Works", step 2).
//
// One wavefront per query row.  Lane l owns projected dims l and l + 64 (d = 128) or dim l
// (d = 64), so that the 64-bit ballot of "dim selected" over the lanes is directly the mask
// word pair of dims 0..63 (and 64..127).
//
// Projection: q'_i = sum_j q_j P[j][i] in fp32, j ascending (fma chain); q_j is broadcast from
// its owner lane with v_readlane.  The workgroup first stages all of P in LDS with 16-byte
// loads (one round trip to L2 instead of one per row j), then each wavefront reads P's rows
// from LDS (consecutive lanes, consecutive banks).
//
// Selection: wave_topk_threshold (exact comparison of sign-cleared fp32 bit patterns, ties to
// the lower index; the k-th largest key built MSB first from wave ballots, stopping as soon as
// exactly k keys clear the running threshold).
#include "aqua_internal.h"

namespace aqua {
namespace {

template <typename QT, int D>
__global__ __launch_bounds__(256) void select_kernel(const QT *__restrict__ q, int N,
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

  const QT *qr = q + static_cast<size_t>(row) * D;
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = load_elem<QT>(qr + lane + 64 * e);

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

  // ---- outputs
  uint64_t sb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sb[e] = __ballot(sel[e]);
  if (q_proj) {
#pragma unroll
    for (int e = 0; e < E; ++e) q_proj[static_cast<size_t>(row) * D + lane + 64 * e] = acc[e];
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

}  // namespace

hipError_t launch_select(const void *q, int qdt, int N, int d, const float *P, int d_sel, int k,
                         float *q_proj, uint32_t *mask, int16_t *idx, hipStream_t s) {
  const dim3 grid((N + 3) / 4), block(256);
  if (qdt == 0 && d == 128)
    select_kernel<float, 128><<<grid, block, 0, s>>>(static_cast<const float *>(q), N, P, d_sel,
                                                     k, q_proj, mask, idx);
  else if (qdt == 0 && d == 64)
    select_kernel<float, 64><<<grid, block, 0, s>>>(static_cast<const float *>(q), N, P, d_sel,
                                                    k, q_proj, mask, idx);
  else if (qdt == 1 && d == 128)
    select_kernel<bf16_t, 128><<<grid, block, 0, s>>>(static_cast<const bf16_t *>(q), N, P,
                                                      d_sel, k, q_proj, mask, idx);
  else
    select_kernel<bf16_t, 64><<<grid, block, 0, s>>>(static_cast<const bf16_t *>(q), N, P,
                                                     d_sel, k, q_proj, mask, idx);
  return hipGetLastError();
}

}  // namespace aqua
