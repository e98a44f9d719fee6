// Causal chunked prefill with per-query dimension selection (AQUA's online step applied to a
// chunk of queries: digest of arXiv 2509.11155, section 方法详解 / 技术框架; edgentiq blog, "How
// AQUA Works", step 2).  Each query keeps its own top-k dims of q' = q P and attends every key at
// a position <= its own.
//
// Two launches per chunk:
//  1. prefill_select_kernel: q' (an fp32-accurate projection on MFMA) and the top-k mask of every
//     query (the selection rule of aqua_select_dims), written out as the MFMA operand: the
//     selected q' dims, pre-multiplied by scale * log2(e), rounded to bf16, zeros elsewhere.
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
// q' = q P on bf16 MFMA at fp32 accuracy: q is bf16, and every fp32 entry of P is the exact sum
// of three bf16 parts (RNE of P, of the remainder, of the remainder's remainder: 8 + 8 + 8
// significand bits), so q' = q P_hi + q P_mid + q P_lo with every product exact and fp32
// accumulation.  A workgroup walks blocks of 32 rows; wavefront w computes output columns
// [32w, 32w + 32) with its parts of P held in registers, writes its q' tile to LDS, and after one
// barrier each wavefront selects 8 of the 32 rows (one row at a time, lane l holding dims l and
// l + 64).
constexpr int SQS = 128 + 8;  // LDS row stride (floats) of the q' tile

__device__ __forceinline__ void split3(float p, uint32_t &h, uint32_t &m, uint32_t &l) {
  h = f32_to_bf16_rne(p);
  const float r1 = p - bf16_to_f32(static_cast<uint16_t>(h));
  m = f32_to_bf16_rne(r1);
  const float r2 = r1 - bf16_to_f32(static_cast<uint16_t>(m));
  l = f32_to_bf16_rne(r2);
}

__global__ __launch_bounds__(256) void prefill_select_kernel(const bf16_t *__restrict__ q, int N,
                                                             const float *__restrict__ P,
                                                             int d_sel, int k, float qscale,
                                                             float *__restrict__ q_proj,
                                                             uint32_t *__restrict__ mask,
                                                             bf16_t *__restrict__ qm) {
  __shared__ __align__(16) float sQ[2][32 * SQS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = 32 * w + (lane & 31);
  // B operands: P[16 m + 8 (lane / 32) + e][col], e = 0..7, in three bf16 parts
  u32x4_t bh[8], bm[8], bl[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    uint32_t h[8], mi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      split3(P[(16 * m + 8 * (lane >> 5) + e) * 128 + col], h[e], mi[e], lo[e]);
    bh[m] = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
    bm[m] = u32x4_t{mi[0] | mi[1] << 16, mi[2] | mi[3] << 16, mi[4] | mi[5] << 16,
                    mi[6] | mi[7] << 16};
    bl[m] = u32x4_t{lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16,
                    lo[6] | lo[7] << 16};
  }
  const int nblk = (N + 31) / 32;
  int buf = 0;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x, buf ^= 1) {
    const int r0 = blk * 32;
    // ---- projection: rows r0 .. r0+31 (clamped), columns [32w, 32w+32)
    const int arow = min(r0 + (lane & 31), N - 1);
    const bf16_t *qa = q + static_cast<size_t>(arow) * 128 + 8 * (lane >> 5);
    u32x4_t av[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) av[m] = *reinterpret_cast<const u32x4_t *>(qa + 16 * m);
    f32x16_t acc_h, acc_l;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc_h[r] = 0.0f;
      acc_l[r] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av[m]);
      acc_l = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bl[m]),
                                                      acc_l, 0, 0, 0);
      acc_l = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bm[m]),
                                                      acc_l, 0, 0, 0);
      acc_h = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bh[m]),
                                                      acc_h, 0, 0, 0);
    }
    float *tile = sQ[buf];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      tile[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SQS + col] = acc_h[r] + acc_l[r];
    __syncthreads();
    // ---- selection: wavefront w takes rows 8w .. 8w+7 of the block
    for (int rr = 8 * w; rr < 8 * w + 8; ++rr) {
      const int row = r0 + rr;
      if (row >= N) break;  // uniform over the wavefront
      const float x[2] = {tile[rr * SQS + lane], tile[rr * SQS + lane + 64]};
      bool sel[2];
      wave_topk_threshold<2>(x, d_sel, k, sel);
      const uint64_t s0 = __ballot(sel[0]), s1 = __ballot(sel[1]);
      if (lane < 4) {
        const uint64_t bb = (lane >> 1) ? s1 : s0;
        mask[static_cast<size_t>(row) * 4 + lane] =
            (lane & 1) ? static_cast<uint32_t>(bb >> 32) : static_cast<uint32_t>(bb);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const size_t at = static_cast<size_t>(row) * 128 + lane + 64 * e;
        if (q_proj) q_proj[at] = x[e];
        qm[at] = sel[e] ? f32_to_bf16_rne(x[e] * qscale) : static_cast<bf16_t>(0);
      }
    }
    // the next block writes the other tile; the barrier above it orders this block's reads
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
  const int nblk = static_cast<int>((rows + 31) / 32);
  prefill_select_kernel<<<dim3(nblk < 512 ? nblk : 512), dim3(256), 0, s>>>(
      static_cast<const bf16_t *>(q), static_cast<int>(rows), P, d_sel, k,
      scale * 1.4426950408889634f, q_proj_out, mask, qm);
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
