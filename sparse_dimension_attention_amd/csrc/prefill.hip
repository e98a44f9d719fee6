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
// One workgroup = 8 wavefronts over the query heads of one KV group (256 query rows), so a
// K'/V tile of 64 tokens is staged in LDS once for all of them.
#include "aqua_internal.h"

namespace aqua {
namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// Waits until no vector memory operation of this wavefront is outstanding (vmcnt(0); the LDS and
// export counters are left alone); memory accesses are not moved across it.  s_waitcnt fields on
// gfx9: vmcnt bits [3:0] and [15:14] (0 here), expcnt [6:4] (7: no wait), lgkmcnt [11:8] (15: no
// wait).
__device__ __forceinline__ void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ 1. selection
// q' = q P with the library's one bf16 projection (proj_mfma: v_mfma_f32_16x16x32_bf16 on P's
// exact three-part bf16 split, fp32 accumulation; the q' of aqua_select_dims bit for bit).  A
// workgroup of 8 wavefronts walks blocks of 32 rows; wavefront w computes output columns
// [16w, 16w + 16), its parts of P held in registers, and writes its part of the q' tile to LDS;
// after one barrier each wavefront selects 4 of the 32 rows (one row at a time, lane l holding
// dims l and l + 64).  The selection is a latency-bound chain of ballots and scalar steps per
// row, so the layout keeps the registers low (16 columns' parts of P per wavefront) for four
// wavefronts per SIMD.
constexpr int SQS = 128 + 8;  // LDS row stride (floats) of the q' tile
constexpr int SEL_WAVES = 8;  // wavefronts per selection workgroup
constexpr int SEL_ROWS_PER_WAVE = 32 / SEL_WAVES;

__global__ __launch_bounds__(SEL_WAVES * 64) void prefill_select_kernel(
    const bf16_t *__restrict__ q, int N, const float *__restrict__ P, int d_sel, int k,
    float qscale, float *__restrict__ q_proj, uint32_t *__restrict__ mask,
    bf16_t *__restrict__ qm) {
  constexpr int R = SEL_ROWS_PER_WAVE;
  __shared__ __align__(16) float sQ[2][32 * SQS];
  __shared__ __align__(16) bf16_t sM[SEL_WAVES * R * 128];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = 16 * w + (lane & 15);
  PParts<4> pp;  // B operands: P's three parts for output columns [16 w, 16 w + 16)
  load_p_parts<4>(P, 16 * w, pp);
  const int nblk = (N + 31) / 32;
  bf16_t *qrows = sM + R * 128 * w;  // this wavefront's rows of qm, staged for 16-byte stores
  // A operands of a block (two halves of 16 rows); each block then loads the next one's before
  // selecting
  u32x4_t av[2][4];
  auto load_rows = [&](int blk) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      load_a_row<4>(q + static_cast<size_t>(min(blk * 32 + 16 * hf + (lane & 15), N - 1)) * 128,
                    av[hf]);
  };
  if (blockIdx.x < nblk) load_rows(blockIdx.x);
  // The rows of each block are waited for explicitly, before the previous block's stores are
  // issued, so the projection needs no wait of its own: the counter of outstanding vector
  // memory operations counts stores too, and a wait placed in the projection could not tell
  // the rows from the stores issued after them.
  wait_vmem();
  int buf = 0;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x, buf ^= 1) {
    const int r0 = blk * 32;
    // ---- projection: rows r0 .. r0+31 (clamped), columns [16w, 16w+16)
    float *tile = sQ[buf];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4_t x = proj_mfma<4>(av[hf], pp);
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[(16 * hf + 4 * (lane >> 4) + r) * SQS + col] = x[r];
    }
    if (blk + static_cast<int>(gridDim.x) < nblk) load_rows(blk + gridDim.x);
    lds_barrier();  // the next block's rows stay in flight through the selection
    // ---- selection: wavefront w takes rows R w .. R w + R - 1 of the block; the masks and q'
    // are held until the next block's rows have landed, then stored
    const int nrows = min(R, N - (r0 + R * w));  // uniform over the wavefront
    uint64_t sm[R][2];
    float xq[R][2];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      sm[rr][0] = sm[rr][1] = 0;
      xq[rr][0] = xq[rr][1] = 0.0f;
      if (rr < nrows) {
        const float *tr = tile + (R * w + rr) * SQS;
        const float x[2] = {tr[lane], tr[lane + 64]};
        bool sel[2];
        wave_topk_threshold<2>(x, d_sel, k, sel);
        sm[rr][0] = __ballot(sel[0]);
        sm[rr][1] = __ballot(sel[1]);
        xq[rr][0] = x[0];
        xq[rr][1] = x[1];
        const uint32_t pair =
            pack_bf16x2(sel[0] ? x[0] * qscale : 0.0f, sel[1] ? x[1] * qscale : 0.0f);
        qrows[rr * 128 + lane] = static_cast<bf16_t>(pair & 0xffffu);
        qrows[rr * 128 + lane + 64] = static_cast<bf16_t>(pair >> 16);
      }
    }
    wait_vmem();  // the next block's rows: requested before the selection, landed by now
    if (nrows > 0) {
      const size_t row0 = static_cast<size_t>(r0 + R * w);
      // masks of the wavefront's rows, contiguous: lane 4 rr + j holds word j of row rr
      if (lane < 4 * nrows) {
        const int j = lane & 3;
        uint32_t word = 0;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const uint32_t w0 = static_cast<uint32_t>(sm[rr][0]);
          const uint32_t w1 = static_cast<uint32_t>(sm[rr][0] >> 32);
          const uint32_t w2 = static_cast<uint32_t>(sm[rr][1]);
          const uint32_t w3 = static_cast<uint32_t>(sm[rr][1] >> 32);
          const uint32_t v = j == 0 ? w0 : (j == 1 ? w1 : (j == 2 ? w2 : w3));
          word = (lane >> 2) == rr ? v : word;
        }
        __builtin_nontemporal_store(word, mask + row0 * 4 + lane);
      }
      if (q_proj) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
          if (rr < nrows) {
            q_proj[(row0 + rr) * 128 + lane] = xq[rr][0];
            q_proj[(row0 + rr) * 128 + lane + 64] = xq[rr][1];
          }
      }
      // the wavefront's rows of qm are contiguous in HBM: 16-byte streaming stores (LDS is in
      // order within a wavefront, so the values written above are read back here)
      bf16_t *dst = qm + row0 * 128;
      const int c = lane;  // 16-byte chunk: row c / 16
      if (c < nrows * 16)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t *>(qrows + 8 * c),
                                    reinterpret_cast<u32x4_t *>(dst + 8 * c));
    }
    // the next block writes the other tile; the barrier above it orders this block's reads
  }
}

// ------------------------------------------------------------------ 2. attention
// A workgroup holds 256 query rows: QB 32-row MFMA blocks per wavefront times NW wavefronts
// (QB * NW = 8).  The launched form is QB = 1, NW = 8: two wavefronts per SIMD, each owning 32
// consecutive positions of one head.  The wavefronts cover the heads of one KV group (or, for
// G < 4, several position blocks), so each 64-token K'/V tile is staged in LDS once for the 256
// rows.
//
// Each wavefront is software-pipelined over the tiles: the scores S of the next tile are computed
// on the matrix cores while the VALU turns the current tile's scores into probabilities, and P V
// of the current tile follows.  So step t reads K' tile t+1 and V tile t; each kind rotates
// through two LDS buffers, and the tiles written in step t (K' t+2, V t+1) replace ones last read
// before the previous barrier: one barrier per tile.  The global loads of the tiles two (K') and
// one (V) ahead are in flight across the step.  Scores come out of the MFMA already relative to
// the row's running max m (the first MFMA of each accumulation chain starts from C = -m), so the
// softmax needs no subtraction; m is checked once per tile, at the end of the step that computed
// its scores, and moves only past a slack (lazy rescale of O and the row sum).  (QB = 2, NW = 4 --
// one wavefront per SIMD, every operand read feeding two MFMAs -- measured slower: with one
// wavefront per SIMD the LDS latencies are exposed.)
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
  int pair;          // 1: a workgroup pairs 32-row block j with block Lq/32 - 1 - j (see below)
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ bf16x8_t lds_tr_pair(const bf16_t *p0, const bf16_t *p1) {
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p0));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p1));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// QB: 32-row query blocks per wavefront; NW: wavefronts per workgroup (QB * NW = 8).
template <int QB, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int ROWS = 32 * QB, NT = NW * 64, CPT = 1024 / NT;
  __shared__ __align__(16) bf16_t sK[2][KBUF];  // K' tiles, [dim][token]
  __shared__ __align__(16) bf16_t sV[2][VBUF];  // V tiles, [token][dim]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int WPH = NW / a.qh;
  const int nsub = G / a.qh;
  const int ncombo = a.B * a.Hkv * nsub;
  const int combo = blockIdx.x % ncombo;
  const int qblk = a.nqb - 1 - blockIdx.x / ncombo;
  const int sub = combo % nsub;
  const int bg = combo / nsub;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int head = g * G + sub * a.qh + (w % a.qh);
  // Paired form (two wavefronts per head, ROWS = 32, Lq a multiple of 64): the head's two
  // wavefronts take 32-row blocks j and Lq / 32 - 1 - j, so every workgroup has about the same
  // causal work; the wavefront of the early block stops computing after its own last tile and
  // the other one, alone on its SIMD from then on, runs faster.  Otherwise the workgroup's
  // wavefronts take consecutive blocks.
  const int pb = a.pair ? (w / a.qh == 0 ? qblk : a.Lq / ROWS - 1 - qblk)
                        : qblk * WPH + w / a.qh;
  const int kend = a.pair ? a.pos0 + a.Lq - qblk * ROWS
                          : a.pos0 + min((qblk + 1) * WPH * ROWS, a.Lq);
  const int ntile = (kend + KT - 1) / KT;
  const int pos_first_wg =
      a.pos0 + (a.pair ? qblk * ROWS : min(qblk * WPH * ROWS, a.Lq - 1));
  // tiles [0, n_pipe) are visible to every row of the workgroup and have a successor: they take
  // the step without causal masking
  const int n_pipe = min((pos_first_wg + 1) / KT, ntile - 1);
  // tiles [0, ntile_w) hold keys this wavefront's rows attend (uniform over the wavefront)
  const int ntile_w = (a.pos0 + min((pb + 1) * ROWS, a.Lq) + KT - 1) / KT;

  int pos[QB], pos_blk[QB];
  u32x4_t qreg[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rl = min(pb * ROWS + qb * 32 + (lane & 31), a.Lq - 1);
    pos[qb] = a.pos0 + rl;
    pos_blk[qb] = a.pos0 + min(pb * ROWS + qb * 32, a.Lq - 1);
    const bf16_t *qr = a.qm + ((static_cast<size_t>(b) * a.Hq + head) * a.Lq + rl) * 128 +
                       8 * (lane >> 5);
#pragma unroll
    for (int m = 0; m < 8; ++m) qreg[qb][m] = *reinterpret_cast<const u32x4_t *>(qr + 16 * m);
  }

  // staging through buffer loads: the descriptors' sizes end K' at d_store dims and V at kend
  // tokens, and reads past a size return zeros (unwritten V is never multiplied by a zero weight;
  // the loads of tiles past the last one read zeros or unused K' and are never consumed)
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(a.kp + static_cast<size_t>(bg) * a.d_store * a.T_cap), (short)0,
      a.d_store * a.T_cap * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(a.v + static_cast<size_t>(bg) * a.T_cap * 128), (short)0, kend * 256,
      0x00020000);
  const int kdim = tid >> 3, kpart = tid & 7;   // K' rows kdim + (NT/8) i, 8 tokens at 8 kpart
  const int vtok = tid >> 4, vpart = tid & 15;  // V rows vtok + (NT/16) i, 8 dims at 8 vpart
  u32x4_t stK[CPT], stV[CPT];
  auto load_K = [&](int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      stK[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rK, (kdim + (NT / 8) * i) * a.T_cap * 2 + 16 * kpart, t * KT * 2, 0);
  };
  auto load_V = [&](int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      stV[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rV, (vtok + (NT / 16) * i) * 256 + 16 * vpart, t * KT * 256, 0);
  };
  auto store_K = [&](bf16_t *dst) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *reinterpret_cast<u32x4_t *>(&dst[(kdim + (NT / 8) * i) * KROW + 8 * kpart]) = stK[i];
  };
  auto store_V = [&](bf16_t *dst) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *reinterpret_cast<u32x4_t *>(&dst[(vtok + (NT / 16) * i) * VROW + 8 * vpart]) = stV[i];
  };
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS traffic done; global loads stay in flight
    __builtin_amdgcn_s_barrier();
  };

  const int g16 = (lane >> 4) & 3, s16 = lane & 15;
  const int k_off = (8 * (g16 >> 1) + (s16 >> 2)) * KROW + 16 * (g16 & 1) + 4 * (s16 & 3);
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
  float m_i[QB], l_i[QB];  // running max (set from the first tile) and row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) l_i[qb] = 0.0f;

  // S^T of 32 tokens (half tb of the tile in kt) for both query blocks
  // scores relative to the running max: the chain's first MFMA adds them to C = -m
  f32x16_t negm[QB];
  auto s_half = [&](const bf16_t *kt, int tb, f32x16_t (&s)[QB]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const bf16_t *p = kt + k_off + 16 * m * KROW + 32 * tb;
      const bf16x8_t av = lds_tr_pair(p, p + 4 * KROW);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            av, __builtin_bit_cast(bf16x8_t, qreg[qb][m]), m == 0 ? negm[qb] : s[qb], 0, 0, 0);
    }
  };
  auto mask_half = [&](int tok0, f32x16_t (&s)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (tok0 + 31 > pos_blk[qb]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = tok0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (tok > pos[qb]) s[qb][r] = -INFINITY;
        }
      }
  };
  // s0, s1 hold a tile's scores relative to m.  A row whose maximum passes the slack moves m up
  // by that maximum: O and l are rescaled, the tile's scores and -m shift with it, and so do the
  // next tile's scores n0, n1 when they were already computed against the old m (shift_next).
  auto rescale = [&](f32x16_t (&s0)[QB], f32x16_t (&s1)[QB], f32x16_t (&n0)[QB],
                     f32x16_t (&n1)[QB], bool shift_next) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = __builtin_fmaxf(s0[qb][0], s0[qb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2)
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[qb][r]), s0[qb][r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, s1[qb][r]), s1[qb][r + 1]);
      if (__ballot(mx > RESCALE_SLACK)) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                         __float_as_uint(mx), false, false);
        mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float dm = mx > RESCALE_SLACK ? mx : 0.0f;
        const float alpha = __builtin_amdgcn_exp2f(-dm);
        l_i[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[qb][db][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[qb][r] -= dm;
          s1[qb][r] -= dm;
        }
        if (shift_next) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            n0[qb][r] -= dm;
            n1[qb][r] -= dm;
          }
        }
        m_i[qb] += dm;
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[qb][r] = -m_i[qb];
      }
    }
  };
  // probabilities as bf16 B operands: pk[qb][16-token step][pair]; the row sum takes the
  // rounded weights, the ones P V multiplies
  uint32_t pk[QB][4][4];
  auto probs = [&](f32x16_t (&s)[QB], int h) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r0 = 8 * ss + 2 * x;
          pk[qb][2 * h + ss][x] = pack_bf16x2(__builtin_amdgcn_exp2f(s[qb][r0]),
                                              __builtin_amdgcn_exp2f(s[qb][r0 + 1]));
          l_i[qb] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2_t, pk[qb][2 * h + ss][x]), ones, l_i[qb], false);
        }
  };
  auto pv_half = [&](const bf16_t *vt, int tb) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t *p = vt + v_off + (32 * tb + 16 * ss) * VROW + 32 * db;
        const bf16x8_t av = lds_tr_pair(p, p + 8 * VROW);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const uint32_t *pq = pk[qb][2 * tb + ss];
          const u32x4_t bv = {pq[0], pq[1], pq[2], pq[3]};
          acc_o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              av, __builtin_bit_cast(bf16x8_t, bv), acc_o[qb][db], 0, 0, 0);
        }
      }
  };

  // One step per tile: the next tile's scores run on the matrix cores while the VALU turns the
  // current tile's into probabilities and P V follows; the next tile's max is checked at the end
  // of the step, next to the barrier.  K' tile t+1 and V tile t are read in step t.
  f32x16_t a0[QB], a1[QB], b0[QB], b1[QB];
  // Past its own last tile a wavefront only helps stage the tiles (masked steps only: every
  // wavefront holds keys in the unmasked ones).
  auto step = [&](int t, f32x16_t (&s0)[QB], f32x16_t (&s1)[QB], f32x16_t (&x0)[QB],
                  f32x16_t (&x1)[QB], bool masked, bool has_next, bool check_next) {
    const bf16_t *vt = sV[t & 1];
    const bool cur = !masked || t < ntile_w;
    const bool nxt = has_next && (!masked || t + 1 < ntile_w);
    if (nxt) {
      s_half(sK[(t + 1) & 1], 0, x0);
      s_half(sK[(t + 1) & 1], 1, x1);
    }
    if (cur) {
      if (masked) {
        mask_half(t * KT, s0);
        mask_half(t * KT + 32, s1);
        rescale(s0, s1, x0, x1, nxt);  // x0, x1 were computed against the m before this tile
      }
      probs(s0, 0);
      probs(s1, 1);
      pv_half(vt, 0);
      pv_half(vt, 1);
    }
    if (check_next) rescale(x0, x1, x0, x1, false);
    store_K(sK[t & 1]);
    store_V(sV[(t + 1) & 1]);
    load_K(t + 3);
    load_V(t + 2);
    barrier();
  };

  load_K(0);
  load_V(0);
  store_K(sK[0]);
  store_V(sV[0]);
  load_K(1);
  store_K(sK[1]);
  load_K(2);
  load_V(1);
  barrier();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[qb][r] = 0.0f;
  s_half(sK[0], 0, a0);
  s_half(sK[0], 1, a1);
  mask_half(0, a0);
  mask_half(32, a1);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {  // every row sees token 0: its max is finite
    float mx = a0[qb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, a0[qb][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, a1[qb][r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    m_i[qb] = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      a0[qb][r] -= m_i[qb];
      a1[qb][r] -= m_i[qb];
      negm[qb][r] = -m_i[qb];
    }
  }
  barrier();  // sK[0] is rewritten in the first step

  int t = 0;
  for (; t + 2 <= n_pipe; t += 2) {
    step(t, a0, a1, b0, b1, false, true, true);
    step(t + 1, b0, b1, a0, a1, false, true, t + 2 < n_pipe);
  }
  for (; t + 2 < ntile; t += 2) {  // causal masking, both tiles with a successor
    step(t, a0, a1, b0, b1, true, true, false);
    step(t + 1, b0, b1, a0, a1, true, true, false);
  }
  for (; t < ntile; ++t) {  // the last tiles: causal masking, and a tile without successor
    step(t, a0, a1, b0, b1, true, t + 1 < ntile, false);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      a0[qb] = b0[qb];
      a1[qb] = b1[qb];
    }
  }

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
  prefill_select_kernel<<<dim3(nblk < 768 ? nblk : 768), dim3(SEL_WAVES * 64), 0, s>>>(
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
  a.pair = (a.qh == 4 && Lq % 64 == 0) ? 1 : 0;  // two 32-row blocks per head and workgroup
  const int grid = a.nqb * (G / a.qh) * B * Hkv;
  prefill_attn_kernel<1, 8><<<dim3(grid), dim3(512), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace aqua
