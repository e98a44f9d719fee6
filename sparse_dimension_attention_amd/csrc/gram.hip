// Gram matrix of calibration vectors, G = X^T X (X [n][d], rows are samples), for AQUA's offline
// projection: P's columns are the right singular vectors of the calibration set, i.e. the
// eigenvectors of G in decreasing order of eigenvalue (digest of arXiv 2509.11155, section
// 方法详解 / 技术框架: the projection comes from an SVD on a calibration set; edgentiq blog,
// "How AQUA Works", step 1).  The O(n d^2) part runs here; the d x d eigensolve is left to the
// caller.
//
// A workgroup takes a chunk of kGC samples and stages it in LDS transposed, dimension-major, as
// bf16 parts: bf16 input as it is; fp32 input as the exact three-part bf16 split of every value
// (split3), so every product of two parts is exact in fp32.  Its 8 wavefronts then compute the
// chunk's G on v_mfma_f32_16x16x32_bf16 (A: 16 dims x 32 samples, B: 32 samples x 16 dims, both
// read as 8 consecutive samples of one dim, one 16-byte LDS read), 9 part products per step for
// fp32 input, fp32 accumulation, and store it as one fp32 partial.  A second kernel adds the
// chunks' partials in fp64.  The only rounding is each chunk's fp32 accumulation (at most kGC or
// 9 kGC terms per entry) and the final fp64 sum.
#include "aqua.h"
#include "aqua_internal.h"

namespace aqua {
namespace {

constexpr int kGC = 128;        // samples per chunk (workgroup)
constexpr int kGR = kGC + 8;    // LDS row stride (bf16) of the transposed chunk

template <typename KT, int D>
__global__ __launch_bounds__(512) void gram_partials_kernel(const KT *__restrict__ x, int64_t n,
                                                            float *__restrict__ part) {
  constexpr int NPART = sizeof(KT) == 4 ? 3 : 1;
  constexpr int NB = D / 16;                // 16-dim blocks per side
  constexpr int BPW = NB * NB / 8;          // output blocks per wavefront
  static_assert(NB * NB % 8 == 0, "blocks per wavefront");
  __shared__ __align__(16) bf16_t sT[NPART][D][kGR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kGC;
  const int ns = static_cast<int>(n - s0 < kGC ? n - s0 : kGC);

  // ---- stage: thread -> one sample's 4 consecutive dims per step; samples past n are zeros
  constexpr int EPI = 4;                    // elements per item
  constexpr int ITEMS = kGC * D / EPI;
  for (int it = tid; it < ITEMS; it += 512) {
    const int t = it / (D / EPI), d0 = EPI * (it % (D / EPI));
    float v[EPI];
    if (t < ns) {
      const KT *src = x + (s0 + t) * D + d0;
      if constexpr (sizeof(KT) == 4) {
        const float4 f = *reinterpret_cast<const float4 *>(src);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else {
        const uint2 r = *reinterpret_cast<const uint2 *>(src);
        v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x); v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPI; ++e) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < EPI; ++e) {
      if constexpr (sizeof(KT) == 4) {
        uint32_t h, m, l;
        split3(v[e], h, m, l);
        sT[0][d0 + e][t] = static_cast<bf16_t>(h);
        sT[1][d0 + e][t] = static_cast<bf16_t>(m);
        sT[2][d0 + e][t] = static_cast<bf16_t>(l);
      } else {
        sT[0][d0 + e][t] = f32_to_bf16_rne(v[e]);  // exact: v is a bf16 value
      }
    }
  }
  __syncthreads();

  // ---- the chunk's G: wavefront w takes output blocks w BPW .. w BPW + BPW - 1 (row-major)
  const int r16 = lane & 15, k8 = 8 * (lane >> 4);
#pragma unroll
  for (int q = 0; q < BPW; ++q) {
    const int blk = w * BPW + q, bi = blk / NB, bj = blk % NB;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kGC / 32; ++ks) {
#pragma unroll
      for (int pa = 0; pa < NPART; ++pa) {
        const bf16x8_t av = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t *>(&sT[pa][16 * bi + r16][32 * ks + k8]));
#pragma unroll
        for (int pb = 0; pb < NPART; ++pb) {
          const bf16x8_t bv = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t *>(&sT[pb][16 * bj + r16][32 * ks + k8]));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
        }
      }
    }
    // D register r: row 4 (l / 16) + r of the block (dim 16 bi + ..), column l % 16
    float *dst = part + static_cast<size_t>(blockIdx.x) * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dst[static_cast<size_t>(16 * bi + 4 * (lane >> 4) + r) * D + 16 * bj + r16] = acc[r];
  }
}

// G[i][j] = the chunks' partials added in fp64, chunk by chunk in order (loads 8 chunks ahead).
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float *__restrict__ part,
                                                          int nchunk, double *__restrict__ g) {
  constexpr int U = 8;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const float *p = part + e;
  double s = 0.0;
  int c = 0;
  for (; c + U <= nchunk; c += U) {
    float v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = p[static_cast<size_t>(c + j) * D * D];
#pragma unroll
    for (int j = 0; j < U; ++j) s += static_cast<double>(v[j]);
  }
  for (; c < nchunk; ++c) s += static_cast<double>(p[static_cast<size_t>(c) * D * D]);
  g[e] = s;
}

template <typename KT, int D>
hipError_t launch_gram_t(const void *x, int64_t n, double *g, void *ws, hipStream_t s) {
  const int nchunk = static_cast<int>((n + kGC - 1) / kGC);
  float *part = static_cast<float *>(ws);
  gram_partials_kernel<KT, D><<<dim3(nchunk), dim3(512), 0, s>>>(static_cast<const KT *>(x), n,
                                                                 part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gram_reduce_kernel<D><<<dim3((D * D + 255) / 256), dim3(256), 0, s>>>(part, nchunk, g);
  return hipGetLastError();
}

}  // namespace

size_t gram_workspace_bytes(int64_t n, int d) {
  const size_t nchunk = static_cast<size_t>((n + kGC - 1) / kGC);
  return nchunk * static_cast<size_t>(d) * d * sizeof(float);
}

hipError_t launch_gram(int dtype, const void *x, int64_t n, int d, double *g, void *ws,
                       hipStream_t s) {
  if (dtype == AQUA_BF16)
    return d == 128 ? launch_gram_t<bf16_t, 128>(x, n, g, ws, s)
                    : launch_gram_t<bf16_t, 64>(x, n, g, ws, s);
  return d == 128 ? launch_gram_t<float, 128>(x, n, g, ws, s)
                  : launch_gram_t<float, 64>(x, n, g, ws, s);
}

}  // namespace aqua
