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
  const uint32_t hm = pack_bf16x2(p, 0.0f);
  h = hm & 0xffffu;
  const float r1 = p - bf16_to_f32(static_cast<uint16_t>(h));
  m = pack_bf16x2(r1, 0.0f) & 0xffffu;
  const float r2 = r1 - bf16_to_f32(static_cast<uint16_t>(m));
  l = pack_bf16x2(r2, 0.0f) & 0xffffu;
}

__global__ __launch_bounds__(256) void prefill_select_kernel(const bf16_t *__restrict__ q, int N,
                                                             const float *__restrict__ P,
                                                             int d_sel, int k, float qscale,
                                                             float *__restrict__ q_proj,
                                                             uint32_t *__restrict__ mask,
                                                             bf16_t *__restrict__ qm) {
  __shared__ __align__(16) float sQ[2][32 * SQS];
  __shared__ __align__(16) bf16_t sM[4 * 8 * 128];
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
  bf16_t *qrows = sM + 8 * 128 * w;  // this wavefront's 8 rows of qm, staged for 16-byte stores
  // A operands of the first block; each block then loads the next one's before selecting
  u32x4_t av[8];
  auto load_rows = [&](int blk) {
    const int arow = min(blk * 32 + (lane & 31), N - 1);
    const bf16_t *qa = q + static_cast<size_t>(arow) * 128 + 8 * (lane >> 5);
#pragma unroll
    for (int m = 0; m < 8; ++m) av[m] = *reinterpret_cast<const u32x4_t *>(qa + 16 * m);
  };
  if (blockIdx.x < nblk) load_rows(blockIdx.x);
  int buf = 0;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x, buf ^= 1) {
    const int r0 = blk * 32;
    // ---- projection: rows r0 .. r0+31 (clamped), columns [32w, 32w+32)
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
    if (blk + static_cast<int>(gridDim.x) < nblk) load_rows(blk + gridDim.x);
    __syncthreads();
    // ---- selection: wavefront w takes rows 8w .. 8w+7 of the block
    const int nrows = min(8, N - (r0 + 8 * w));  // uniform over the wavefront
    for (int rr = 0; rr < nrows; ++rr) {
      const int row = r0 + 8 * w + rr;
      const float *tr = tile + (8 * w + rr) * SQS;
      const float x[2] = {tr[lane], tr[lane + 64]};
      bool sel[2];
      wave_topk_threshold<2>(x, d_sel, k, sel);
      const uint64_t s0 = __ballot(sel[0]), s1 = __ballot(sel[1]);
      if (lane < 4) {
        const uint64_t bb = (lane >> 1) ? s1 : s0;
        mask[static_cast<size_t>(row) * 4 + lane] =
            (lane & 1) ? static_cast<uint32_t>(bb >> 32) : static_cast<uint32_t>(bb);
      }
      if (q_proj) {
        q_proj[static_cast<size_t>(row) * 128 + lane] = x[0];
        q_proj[static_cast<size_t>(row) * 128 + lane + 64] = x[1];
      }
      const uint32_t pair = pack_bf16x2(sel[0] ? x[0] * qscale : 0.0f, sel[1] ? x[1] * qscale : 0.0f);
      qrows[rr * 128 + lane] = static_cast<bf16_t>(pair & 0xffffu);
      qrows[rr * 128 + lane + 64] = static_cast<bf16_t>(pair >> 16);
    }
    // the wavefront's rows of qm are contiguous in HBM: 16-byte stores (LDS is in order within
    // a wavefront, so the values written above are read back here)
    if (nrows > 0) {
      bf16_t *dst = qm + static_cast<size_t>(r0 + 8 * w) * 128;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h;  // 16-byte chunk: row c / 16
        if (c < nrows * 16)
          *reinterpret_cast<u32x4_t *>(dst + 8 * c) =
              *reinterpret_cast<const u32x4_t *>(qrows + 8 * c);
      }
    }
    // the next block writes the other tile; the barrier above it orders this block's reads
  }
}

// ------------------------------------------------------------------ 2. attention
// A workgroup holds 256 query rows: QB 32-row MFMA blocks per wavefront times NW wavefronts
// (QB * NW = 8).  The launched form is QB = 1, NW = 8: two wavefronts per SIMD, each owning 32
// consecutive positions of one head, so one wavefront's softmax can overlap the other's MFMAs;
// QB = 2, NW = 4 (one wavefront per SIMD, every K'/V operand read feeding two MFMAs) measured
// slower.  The wavefronts cover the heads of one KV group (or, for G < 4, several position
// blocks), so each 64-token K'/V tile is staged in LDS once for the 256 rows.  Tiles are
// double-buffered: the global loads of tile t+1 are in flight while tile t is computed, and one
// barrier per tile hands the buffers over.
//
// Operands come out of LDS with ds_read_b64_tr_b16, which within each 16-lane group reads a
// 4-row x 16-column block of 16-bit elements (lane s of the group supplying the address of row
// s / 4, columns 4 (s % 4) .. +3) and hands lane i = 4a + b the column i: element e of its result
// is row e, column i.  So the MFMA A operand (lane l: row l % 32, 8 consecutive k) is read from
// a tile stored k-major, which is how K' ([dim][token]) and V ([token][dim]) already are in HBM:
// the staging is a plain 16-byte copy.
constexpr int KT = 64;          // tokens per tile
constexpr int KROW = KT + 32;   // LDS row (dim) stride of the K' tile, bf16: 192 B
constexpr int VROW = 128 + 32;  // LDS row (token) stride of the V tile, bf16: 320 B
constexpr int KBUF = 128 * KROW;
constexpr int VBUF = KT * VROW;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units the running max may lag the true max

struct PrefillArgs {
  const bf16_t *kp;  // [B][Hkv][d_store][T_cap]
  const bf16_t *v;   // [B][Hkv][T_cap][128]
  const bf16_t *qm;  // [B][Hq][Lq][128] masked, scaled q'
  float *out;        // [B][Hq][Lq][128]
  int B, Hq, Hkv, d_store, T_cap, Lq, pos0;
  int qh;            // query heads per workgroup (min(G, 4))
  int nqb;           // position blocks per (b, group, head subset)
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ bf16x8_t lds_tr_pair(const bf16_t *p0, const bf16_t *p1) {
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p0));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p1));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// QB: 32-row query blocks per wavefront; NW: wavefronts per workgroup (QB * NW = 8, so a
// workgroup always holds 256 query rows).
template <int QB, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int NT = NW * 64;      // threads
  constexpr int CPT = 1024 / NT;   // 16-byte chunks of K' (and of V) staged per thread per tile
  constexpr int ROWS = 32 * QB;    // query rows per wavefront
  __shared__ __align__(16) bf16_t sK[2][KBUF];  // K' tile, [dim][token]
  __shared__ __align__(16) bf16_t sV[2][VBUF];  // V tile, [token][dim]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int WPH = NW / a.qh;    // wavefronts per head: consecutive ROWS-position blocks
  const int nsub = G / a.qh;    // head subsets per KV group
  const int ncombo = a.B * a.Hkv * nsub;
  // consecutive workgroup ids go round-robin over the XCDs: keep one (b, group) per id residue
  // so that the workgroups sharing a K'/V stream share an L2; latest positions first
  const int combo = blockIdx.x % ncombo;
  const int qblk = a.nqb - 1 - blockIdx.x / ncombo;
  const int sub = combo % nsub;
  const int bg = combo / nsub;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int head = g * G + sub * a.qh + (w % a.qh);
  const int pb = qblk * WPH + w / a.qh;  // this wavefront's block of ROWS positions
  const int kend = a.pos0 + min((qblk + 1) * WPH * ROWS, a.Lq);  // keys [0, kend) for the group
  const int ntile = (kend + KT - 1) / KT;

  // ---- the wavefront's query rows (B operand of S^T), one 16-dim step per register group
  int pos[QB];
  u32x4_t qreg[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rl = min(pb * ROWS + qb * 32 + (lane & 31), a.Lq - 1);
    pos[qb] = a.pos0 + rl;
    const bf16_t *qr = a.qm + ((static_cast<size_t>(b) * a.Hq + head) * a.Lq + rl) * 128 +
                       8 * (lane >> 5);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      qreg[qb][m] = *reinterpret_cast<const u32x4_t *>(qr + 16 * m);
      asm volatile("" : "+a"(qreg[qb][m]));  // MFMA B operands only: keep them in AGPRs
    }
  }
  const int pos_first = a.pos0 + min(pb * ROWS, a.Lq - 1);  // earliest row of the wavefront

  // ---- staging through buffer loads: the descriptors' sizes end K' at d_store dims and V at
  // kend tokens, and reads past a size return zeros (never multiply unwritten V by a zero weight)
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(a.kp + static_cast<size_t>(bg) * a.d_store * a.T_cap), (short)0,
      a.d_store * a.T_cap * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(a.v + static_cast<size_t>(bg) * a.T_cap * 128), (short)0, kend * 256,
      0x00020000);
  const int kdim = tid >> 3, kpart = tid & 7;   // K' rows kdim + (NT/8) i, 8 tokens at 8 kpart
  const int vtok = tid >> 4, vpart = tid & 15;  // V rows vtok + (NT/16) i, 8 dims at 8 vpart
  u32x4_t stK[CPT], stV[CPT];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      stK[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rK, (kdim + (NT / 8) * i) * a.T_cap * 2 + 16 * kpart, t0 * 2, 0);
      stV[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rV, (vtok + (NT / 16) * i) * 256 + 16 * vpart, t0 * 256, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      *reinterpret_cast<u32x4_t *>(&sK[buf][(kdim + (NT / 8) * i) * KROW + 8 * kpart]) = stK[i];
      *reinterpret_cast<u32x4_t *>(&sV[buf][(vtok + (NT / 16) * i) * VROW + 8 * vpart]) = stV[i];
    }
  };

  // per-lane parts of the transposed-read addresses (see the comment at the top of this part)
  const int g16 = (lane >> 4) & 3, s16 = lane & 15;
  // K': row (dim) 16 m + 8 (g16 / 2) + 4 j + s16 / 4, column (token) 32 tb + 16 (g16 % 2) + 4 (s16 % 4)
  const int k_off = (8 * (g16 >> 1) + (s16 >> 2)) * KROW + 16 * (g16 & 1) + 4 * (s16 & 3);
  // V: row (token) 32 tb + 16 s + 4 (g16 / 2) + 8 j + s16 / 4, column (dim) 32 db + 16 (g16 % 2) + 4 (s16 % 4)
  const int v_off = (4 * (g16 >> 1) + (s16 >> 2)) * VROW + 16 * (g16 & 1) + 4 * (s16 & 3);

  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16_t acc_o[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[qb][db][r] = 0.0f;
  float m_i[QB], l_i[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_i[qb] = -INFINITY;
    l_i[qb] = 0.0f;
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int buf = t & 1, t0 = t * KT;
    if (t + 1 < ntile) load_tile(t0 + KT);
    const bf16_t *kt = sK[buf] + k_off;
    const bf16_t *vt = sV[buf] + v_off;

#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {  // 32-token halves of the tile, one after the other
      // ---- S^T = K'^T Q'^T for the 32 tokens x QB query blocks
      f32x16_t acc_s[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[qb][r] = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const bf16_t *p = kt + 16 * m * KROW + 32 * tb;
        const bf16x8_t av = lds_tr_pair(p, p + 4 * KROW);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc_s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              av, __builtin_bit_cast(bf16x8_t, qreg[qb][m]), acc_s[qb], 0, 0, 0);
      }

      // ---- causal mask, online softmax (log2 units), probabilities as bf16 B operands
      const int tok0 = t0 + 32 * tb;
      uint32_t pk[QB][2][4];  // [qb][16-token step][packed pair]
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (tok0 + 31 > pos_first + 32 * qb) {  // the block reaches past some row's position
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = tok0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (tok > pos[qb]) acc_s[qb][r] = -INFINITY;
          }
        }
        float mx = acc_s[qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, acc_s[qb][r]);
        {  // lanes l and l ^ 32 hold the two halves of a row's scores
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                           __float_as_uint(mx), false, false);
          mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        // the running max moves only when a score exceeds it by more than the slack, so the
        // probabilities stay <= 2^slack and the rescale of O is rare after the first block
        const bool grow = mx > m_i[qb] + RESCALE_SLACK;
        if (__ballot(grow)) {
          const float m_new = grow ? mx : m_i[qb];
          const float alpha = __builtin_amdgcn_exp2f(m_i[qb] - m_new);
          l_i[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[qb][db][r] *= alpha;
          m_i[qb] = m_new;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r0 = 8 * s + 2 * x;
            pk[qb][s][x] = pack_bf16x2(__builtin_amdgcn_exp2f(acc_s[qb][r0] - m_i[qb]),
                                       __builtin_amdgcn_exp2f(acc_s[qb][r0 + 1] - m_i[qb]));
            // the row sum takes the rounded weights, the ones P V multiplies
            l_i[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[qb][s][x]),
                                                      ones, l_i[qb], false);
          }
      }

      // ---- O^T += V^T P^T over the 32 tokens
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16_t *p = vt + (32 * tb + 16 * s) * VROW + 32 * db;
          const bf16x8_t av = lds_tr_pair(p, p + 8 * VROW);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const u32x4_t bv = {pk[qb][s][0], pk[qb][s][1], pk[qb][s][2], pk[qb][s][3]};
            acc_o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                av, __builtin_bit_cast(bf16x8_t, bv), acc_o[qb][db], 0, 0, 0);
          }
        }
    }

    if (t + 1 < ntile) store_tile(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }

  // ---- normalise and write: lane l owns query row l % 32, dims db*32 + 8(r/4) + 4(l/32) + r%4
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rl = pb * ROWS + qb * 32 + (lane & 31);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_i[qb]),
                                                     __float_as_uint(l_i[qb]), false, false);
    const float inv = 1.0f / (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
    if (rl < a.Lq) {
      float *orow = a.out + ((static_cast<size_t>(b) * a.Hq + head) * a.Lq + rl) * 128;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const float4 vv =
              make_float4(acc_o[qb][db][4 * rq] * inv, acc_o[qb][db][4 * rq + 1] * inv,
                          acc_o[qb][db][4 * rq + 2] * inv, acc_o[qb][db][4 * rq + 3] * inv);
          *reinterpret_cast<float4 *>(orow + db * 32 + 8 * rq + 4 * (lane >> 5)) = vv;
        }
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
  const int rows_per_wg = 256 / a.qh;  // 256 query rows per workgroup over qh heads
  a.nqb = (Lq + rows_per_wg - 1) / rows_per_wg;
  const int grid = a.nqb * (G / a.qh) * B * Hkv;
#ifdef AQUA_PREFILL_QB
  constexpr int QB = AQUA_PREFILL_QB;
#else
  constexpr int QB = 1;
#endif
  prefill_attn_kernel<QB, 8 / QB><<<dim3(grid), dim3(64 * (8 / QB)), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace aqua
