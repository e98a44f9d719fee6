// Causal chunked prefill with per-query dimension selection (AQUA's online step applied to a
// chunk of queries: digest of arXiv 2509.11155, section 方法详解 / 技术框架; edgentiq blog, "How
// AQUA Works", step 2).  Each query keeps its own top-k dims of q' = q P and attends every key at
// a position <= its own.
//
// Two launches per chunk:
//  1. prefill_select_kernel: q' and the top-k mask of every query (the selection of
//     aqua_select_dims, bit-identical), written out as the MFMA operand: the selected q' dims,
//     pre-multiplied by scale * log2(e), rounded to bf16, zeros elsewhere.
//  2. prefill_attn_kernel: flash-attention style on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with
//     fp32 accumulation.  The zeroed dims still cost MFMA work: the dense contraction over all
//     stored dims is the cheapest exact way to apply per-query masks on matrix cores.
//
// MFMA formulation (lane layout of the 32x32x16 bf16 instruction: A lane l holds row l%32,
// k = 8*(l/32)+e; B lane l holds column l%32, same k; D register r holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32):
//  * S^T = K'^T Q'^T: A = K' tile transposed to [token][dim] in LDS, B = the wavefront's 32 query
//    rows (registers, loaded once).  D then holds, in lane l, scores of query row l%32 for 16 of
//    the 32 tokens of a block, so the online softmax statistics of a row live in one lane pair.
//  * O^T = V^T P^T: A = V tile transposed to [dim][token] in LDS, B = the probabilities straight
//    from the S^T registers.  The contraction over tokens is taken in the order the S^T layout
//    hands out (lane l < 32: tokens 0-3, 8-11 of a 16-token step; lane l >= 32: tokens 4-7,
//    12-15), and the V operand is read in that same order.  D holds O^T with lane l owning
//    query row l%32, so the softmax rescale is one scalar per lane.
// One workgroup = 4 wavefronts = 4 (query head, 32-position block) pairs of one KV group, so a
// K'/V tile of 64 tokens is staged once for 4 heads.
#include "aqua_internal.h"

namespace aqua {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ 1. selection
// Each wavefront handles `rpw` consecutive rows; the workgroup stages P in LDS once.
template <typename QT>
__global__ __launch_bounds__(256) void prefill_select_kernel(const QT *__restrict__ q, int N,
                                                             const float *__restrict__ P,
                                                             int d_sel, int k, float qscale,
                                                             int rpw, float *__restrict__ q_proj,
                                                             uint32_t *__restrict__ mask,
                                                             bf16_t *__restrict__ qm) {
  constexpr int D = 128, E = 2;
  __shared__ float sP[D * D];
  {
    constexpr int NV = D * D / (256 * 4);
#pragma unroll
    for (int v0 = 0; v0 < NV; v0 += 4) {
      float4 st[4];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        st[v] = *reinterpret_cast<const float4 *>(&P[((v0 + v) * 256 + threadIdx.x) * 4]);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<float4 *>(&sP[((v0 + v) * 256 + threadIdx.x) * 4]) = st[v];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * rpw;
  for (int rr = 0; rr < rpw; ++rr) {
    const int row = row0 + rr;
    if (row >= N) break;  // uniform over the wavefront; no workgroup barrier follows
    const QT *qr = q + static_cast<size_t>(row) * D;
    float qv[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qv[e] = load_elem<QT>(qr + lane + 64 * e);
      acc[e] = 0.0f;
    }
#pragma unroll 16
    for (int j = 0; j < D; ++j) {
      const float src = (j < 64) ? qv[0] : qv[1];
      const float qj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), j & 63));
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(qj, sP[j * D + lane + 64 * e], acc[e]);
    }
    bool sel[E];
    wave_topk<E>(acc, d_sel, k, sel);
    uint64_t sb[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sb[e] = __ballot(sel[e]);
    if (lane < 4) {
      const uint64_t bb = (lane >> 1) ? sb[1] : sb[0];
      mask[static_cast<size_t>(row) * 4 + lane] =
          (lane & 1) ? static_cast<uint32_t>(bb >> 32) : static_cast<uint32_t>(bb);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const size_t at = static_cast<size_t>(row) * D + lane + 64 * e;
      if (q_proj) q_proj[at] = acc[e];
      qm[at] = sel[e] ? f32_to_bf16_rne(acc[e] * qscale) : static_cast<bf16_t>(0);
    }
  }
}

// ------------------------------------------------------------------ 2. attention
constexpr int KT = 64;          // tokens per K'/V tile
constexpr int KS = 128 + 8;     // LDS row stride (bf16) of the K' tile [token][dim]
constexpr int VS = KT + 4;      // LDS row stride (bf16) of the V tile [dim][token]

struct PrefillArgs {
  const bf16_t *kp;  // [B][Hkv][d_store][T_cap]
  const bf16_t *v;   // [B][Hkv][T_cap][128]
  const bf16_t *qm;  // [B][Hq][Lq][128] masked, scaled q'
  float *out;        // [B][Hq][Lq][128]
  int B, Hq, Hkv, d_store, T_cap, Lq, pos0;
  int qh;            // query heads per workgroup (min(G, 4))
  int nqb;           // query blocks per (b, group, head subset)
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_rne(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_rne(hi)) << 16);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __align__(16) bf16_t sK[KT * KS];   // K' tile, [token][dim]
  __shared__ __align__(16) bf16_t sV[128 * VS];  // V tile, [dim][token]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int PB = 4 / a.qh;                      // 32-position blocks per workgroup
  const int nsub = G / a.qh;                    // head subsets per KV group
  // heaviest (latest positions) first
  const int qblk = a.nqb - 1 - (blockIdx.x % a.nqb);
  const int rest = blockIdx.x / a.nqb;
  const int sub = rest % nsub;
  const int bg = rest / nsub;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int head = g * G + sub * a.qh + (w % a.qh);
  const int pblk = qblk * PB + w / a.qh;
  const int row_local = pblk * 32 + (lane & 31);           // position within the chunk
  const int row_c = min(row_local, a.Lq - 1);
  const int pos = a.pos0 + row_c;                           // absolute position of this row
  const int kend = a.pos0 + min((qblk + 1) * PB * 32, a.Lq);  // keys [0, kend) for the group
  const int nks = a.d_store / 16;

  // the wavefront's 32 query rows as the B operand of S^T, one 16-dim step per register group
  const size_t qrow = (static_cast<size_t>(b) * a.Hq + head) * a.Lq + row_c;
  u32x4_t qreg[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
    qreg[m] = *reinterpret_cast<const u32x4_t *>(a.qm + qrow * 128 + 16 * m + 8 * (lane >> 5));

  f32x16_t acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.0f;
  float m_i = -INFINITY, l_i = 0.0f;

  const bf16_t *kbase = a.kp + static_cast<size_t>(bg) * a.d_store * a.T_cap;
  const bf16_t *vbase = a.v + static_cast<size_t>(bg) * a.T_cap * 128;
  const int ntile = (kend + KT - 1) / KT;

  for (int t = 0; t < ntile; ++t) {
    const int t0 = t * KT;
    // ---- stage K' (dims [0, d_store) x 64 tokens) as [token][dim], V as [dim][token]
    for (int ci = tid; ci < a.d_store * 8; ci += 256) {
      const int d = ci % a.d_store, c = ci / a.d_store;  // consecutive lanes: consecutive dims
      const u32x4_t r = *reinterpret_cast<const u32x4_t *>(
          kbase + static_cast<size_t>(d) * a.T_cap + t0 + 8 * c);
      const uint32_t wds[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sK[(8 * c + 2 * x) * KS + d] = static_cast<bf16_t>(wds[x] & 0xffffu);
        sK[(8 * c + 2 * x + 1) * KS + d] = static_cast<bf16_t>(wds[x] >> 16);
      }
    }
    for (int ci = tid; ci < KT * 16; ci += 256) {
      const int tok = ci % KT, c = ci / KT;  // consecutive lanes: consecutive tokens
      u32x4_t r = {0u, 0u, 0u, 0u};
      if (t0 + tok < kend)  // never multiply garbage V by a zero weight
        r = *reinterpret_cast<const u32x4_t *>(vbase + static_cast<size_t>(t0 + tok) * 128 +
                                               8 * c);
      const uint32_t wds[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sV[(8 * c + 2 * x) * VS + tok] = static_cast<bf16_t>(wds[x] & 0xffffu);
        sV[(8 * c + 2 * x + 1) * VS + tok] = static_cast<bf16_t>(wds[x] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T for two 32-token blocks
    f32x16_t acc_s[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_s[tb][r] = 0.0f;
      const bf16_t *krow = sK + (tb * 32 + (lane & 31)) * KS + 8 * (lane >> 5);
      for (int m = 0; m < nks; ++m) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t *>(krow + 16 * m);
        acc_s[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, qreg[m]), acc_s[tb],
            0, 0, 0);
      }
    }
    // ---- causal mask (token > row position), online softmax in log2 units
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = t0 + tb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (tok > pos) acc_s[tb][r] = -INFINITY;
        mx = fmaxf(mx, acc_s[tb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_i, mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_i - m_new);
    float rs = 0.0f;
    uint32_t pk[2][2][4];  // [tb][k-step][packed pair]
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r0 = 8 * s + 2 * x;
          const float p0 = (m_new == -INFINITY) ? 0.0f
                                                : __builtin_amdgcn_exp2f(acc_s[tb][r0] - m_new);
          const float p1 = (m_new == -INFINITY)
                               ? 0.0f
                               : __builtin_amdgcn_exp2f(acc_s[tb][r0 + 1] - m_new);
          rs += p0 + p1;
          pk[tb][s][x] = pack_bf16x2(p0, p1);
        }
    rs += __shfl_xor(rs, 32, 64);
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16_t *vrow = sV + (db * 32 + (lane & 31)) * VS + 4 * (lane >> 5);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16_t *vp = vrow + tb * 32 + 16 * s;
          const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vp);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vp + 8);
          const u32x4_t av = {lo.x, lo.y, hi.x, hi.y};
          const u32x4_t bv = {pk[tb][s][0], pk[tb][s][1], pk[tb][s][2], pk[tb][s][3]};
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc_o[db], 0,
              0, 0);
        }
    }
    __syncthreads();  // the next tile overwrites the LDS tiles
  }

  // ---- normalise and write: lane l owns query row l%32, dims db*32 + 8*(r/4) + 4*(l/32) + r%4
  if (row_local < a.Lq) {
    const float inv = 1.0f / l_i;
    float *orow = a.out + ((static_cast<size_t>(b) * a.Hq + head) * a.Lq + row_local) * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 vv = make_float4(acc_o[db][4 * rq] * inv, acc_o[db][4 * rq + 1] * inv,
                                      acc_o[db][4 * rq + 2] * inv, acc_o[db][4 * rq + 3] * inv);
        *reinterpret_cast<float4 *>(orow + db * 32 + 8 * rq + 4 * (lane >> 5)) = vv;
      }
  }
}

}  // namespace

size_t prefill_workspace_bytes(int B, int Hq, int Lq) {
  const size_t rows = static_cast<size_t>(B) * Hq * Lq;
  return rows * 128 * 2 + ((rows * 16 + 255) & ~static_cast<size_t>(255));
}

hipError_t launch_prefill(const void *kp, const void *v, int B, int Hq, int Hkv, int d_store,
                          int T_cap, const void *q, int Lq, int pos0, const float *P, int d_sel,
                          int k, float scale, float *out, float *q_proj_out, uint32_t *mask_out,
                          void *ws, hipStream_t s) {
  const size_t rows = static_cast<size_t>(B) * Hq * Lq;
  bf16_t *qm = static_cast<bf16_t *>(ws);
  uint32_t *mask = mask_out ? mask_out : reinterpret_cast<uint32_t *>(qm + rows * 128);
  const int rpw = 8;  // rows per wavefront
  const int nblk = static_cast<int>((rows + 4 * rpw - 1) / (4 * rpw));
  prefill_select_kernel<bf16_t><<<dim3(nblk), dim3(256), 0, s>>>(
      static_cast<const bf16_t *>(q), static_cast<int>(rows), P, d_sel, k,
      scale * 1.4426950408889634f, rpw, q_proj_out, mask, qm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillArgs a;
  a.kp = static_cast<const bf16_t *>(kp);
  a.v = static_cast<const bf16_t *>(v);
  a.qm = qm;
  a.out = out;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d_store = d_store;
  a.T_cap = T_cap;
  a.Lq = Lq;
  a.pos0 = pos0;
  const int G = Hq / Hkv;
  a.qh = G < 4 ? G : 4;
  const int rows_per_wg = 32 * (4 / a.qh);
  a.nqb = (Lq + rows_per_wg - 1) / rows_per_wg;
  const int grid = a.nqb * (G / a.qh) * B * Hkv;
  prefill_attn_kernel<<<dim3(grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace aqua
