// Online key projection into the dimension-major K' cache (AQUA's online step projects keys with
// the offline matrix: digest of arXiv 2509.11155, section 方法详解 / 技术框架; edgentiq blog, "How
// AQUA Works", step 2).  Only dims 0..d_store-1 are kept (AQUA-Memory's static cut, blog section
// "AQUA-Memory").  V is copied unchanged.
//
// bf16 keys take the library's one bf16 projection (proj_mfma: v_mfma_f32_16x16x32_bf16 on P's
// exact three-part bf16 split, fp32 accumulation), so a key's K' is the same bits whichever
// kernel projects it (this one, the fused decode step's, the fused H2O step's).  One workgroup of
// 8 wavefronts per tile of 64 tokens of one (b, g), four workgroups per CU (36 KB of LDS each),
// so that the loads of some overlap the projection and stores of others: wavefront w takes the
// parts of P for its 16 output dims, the tile's keys are staged in LDS (16 bytes per lane,
// coalesced) and its values go from registers straight to the cache; the wavefronts project the
// tile's 16-token blocks, round to bf16 and transpose through LDS, so that each K' row gets 64
// consecutive tokens (128 bytes), written 16 bytes per lane.  (A loop over tiles per workgroup
// with the next tile's loads in flight does not pay here: loads and stores share one in-order
// wait counter, so with a variable number of stores per tile every wait for the next tile's data
// also waits for this tile's stores.)  HBM-bound: 2 d bytes of K read, 2 d_store bytes of
// K' and 4 d bytes of V moved per token.
//
// fp32 keys (the VALU path): tiles of 32 tokens staged in LDS as fp32; thread (i, group) computes
// K'[t][i] = sum_j K[t][j] P[j][i] for its tokens (j ascending, fma), then the same transposed
// write.
#include <algorithm>

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

// ------------------------------------------------------------------ bf16: MFMA
constexpr int kMT = 64;  // tokens per tile (one tile per workgroup)

template <int D>
__global__ __launch_bounds__(512) void project_keys_mfma_kernel(
    const bf16_t *__restrict__ k_raw, const bf16_t *__restrict__ v_raw,
    const float *__restrict__ P, int n, int d_store, int T_cap, int len0,
    const int32_t *__restrict__ slots, bf16_t *__restrict__ kp, bf16_t *__restrict__ vc) {
  constexpr int KS = D / 32, NB = D / 16;
  constexpr int WPB = 8 / NB;      // wavefronts per column block (they split the token blocks)
  constexpr int KR = D + 8;        // LDS row stride (bf16) of the staged key tile
  constexpr int KROW = kMT + 8;    // LDS row stride (bf16) of the transposed tile
  constexpr int PR = D / 8;        // 16-byte pieces per key or value row
  constexpr int CH = kMT * PR / 512;  // pieces of the tile's K (and of its V) per thread
  static_assert(CH >= 1 && kMT * PR % 512 == 0, "tile pieces per thread");
  __shared__ __align__(16) bf16_t ks[kMT][KR];
  __shared__ __align__(16) bf16_t kt[D][KROW];
  __shared__ int cols[kMT];
  const int bg = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int blk = w % NB, tb0 = w / NB;
  const int t0 = blockIdx.x * kMT, nt = min(kMT, n - t0);
  const bf16_t *kb = k_raw + static_cast<size_t>(bg) * n * D;
  // every load is issued before the first wait: P's values, the tile's keys and values (16 bytes
  // per lane, coalesced), the destination columns
  float pv[KS][8];
  load_p_raw<KS>(P, 16 * blk, pv);
  u32x4_t kr[CH], vr[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int pc = tid + 512 * c;
    const size_t off = static_cast<size_t>(min(t0 + pc / PR, n - 1)) * D + 8 * (pc % PR);
    kr[c] = *reinterpret_cast<const u32x4_t *>(kb + off);
    if (v_raw) vr[c] = *reinterpret_cast<const u32x4_t *>(v_raw + static_cast<size_t>(bg) * n * D + off);
  }
  if (tid < kMT) {
    int col = -1;
    if (tid < nt) col = slots ? slots[static_cast<size_t>(bg) * n + t0 + tid] : len0 + t0 + tid;
    cols[tid] = (col >= 0 && col < T_cap) ? col : -1;
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int pc = tid + 512 * c;
    *reinterpret_cast<u32x4_t *>(&ks[pc / PR][8 * (pc % PR)]) = kr[c];
  }
  PParts<KS> pp;
  split_p_parts<KS>(pv, pp);
  __syncthreads();
  // V rows, 16 bytes per lane, straight from registers
  if (v_raw) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int pc = tid + 512 * c, t = pc / PR;
      const int col = cols[t];
      if (t < nt && col >= 0)
        *reinterpret_cast<u32x4_t *>(vc + (static_cast<size_t>(bg) * T_cap + col) * D +
                                     8 * (pc % PR)) = vr[c];
    }
  }
  // K' of the tile: wavefront (blk, tb0) takes 16-token blocks tb0, tb0 + WPB, ...
#pragma unroll
  for (int tb = tb0; tb < kMT / 16; tb += WPB) {
    u32x4_t av[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st)
      av[st] = *reinterpret_cast<const u32x4_t *>(&ks[16 * tb + (lane & 15)]
                                                    [32 * st + 8 * (lane >> 4)]);
    const f32x4_t x = proj_mfma<KS>(av, pp);
    *reinterpret_cast<uint2 *>(&kt[16 * blk + (lane & 15)][16 * tb + 4 * (lane >> 4)]) =
        make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
  __syncthreads();
  // K' rows: chunks of 8 tokens; a chunk whose 8 columns are consecutive and 16-byte aligned is
  // one store, any other is written token by token
  for (int e = tid; e < d_store * (kMT / 8); e += 512) {
    const int row = e / (kMT / 8), ta = 8 * (e % (kMT / 8));
    if (ta >= nt) continue;
    bf16_t *dst = kp + (static_cast<size_t>(bg) * d_store + row) * T_cap;
    const int c0 = cols[ta];
    bool vec = ta + 8 <= nt && c0 >= 0 && (c0 & 7) == 0;
#pragma unroll
    for (int j = 1; j < 8; ++j) vec = vec && cols[ta + j] == c0 + j;
    if (vec) {
      *reinterpret_cast<uint4 *>(dst + c0) = *reinterpret_cast<const uint4 *>(&kt[row][ta]);
    } else {
      for (int j = 0; j < 8 && ta + j < nt; ++j)
        if (cols[ta + j] >= 0) dst[cols[ta + j]] = kt[row][ta + j];
    }
  }
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Bulk append (no slot list, len0 a multiple of 8): each workgroup (about one per CU) streams a
// contiguous run of whole 64-token tiles of one (b, g), its wavefronts' parts of P held in
// registers for the whole run; the last workgroup of each (b, g) then takes the ragged tail.
// Tile i + 3's keys and values are requested before tile i is worked on (four register sets in
// turn, no copies at the loop latch), and every store of a whole tile is unconditional, so that
// each wait is exactly "the next three tiles' loads plus their stores still in flight":
//  * V rows: 16 bytes per lane, from registers, streaming stores;
//  * the keys: through LDS (two buffers, one barrier per tile) into the MFMA A operands;
//  * K': each wavefront's 16 dims x 64 tokens go through a slice of LDS of its own (no barrier)
//    and out as 128 contiguous bytes per K' row, 16 bytes per lane, streaming stores.  Lanes
//    whose dim is at or past d_store compute dim d_store - 1 again and store that same value.
constexpr int kNS = 4;  // register sets: tiles in flight ahead of the one worked on, plus one
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void project_keys_stream_kernel(const bf16_t *__restrict__ k_raw, const bf16_t *__restrict__ v_raw,
                                const float *__restrict__ P, int n, int d_store, int T_cap,
                                int len0, int tiles_per_wg, bf16_t *__restrict__ kp,
                                bf16_t *__restrict__ vc) {
  constexpr int KS = D / 32, NB = D / 16;
  constexpr int WPB = 8 / NB;          // wavefronts per column block (they split the token blocks)
  constexpr int KR = D + 8;            // LDS row stride (bf16) of a staged key tile
  constexpr int TR = kMT + 8;          // LDS row stride (bf16) of a wavefront's K' slice
  constexpr int PR = D / 8;            // 16-byte pieces per key or value row
  constexpr int CH = kMT * PR / 512;   // pieces of a tile's K (and of its V) per thread
  static_assert(CH >= 1 && kMT * PR % 512 == 0, "tile pieces per thread");
  static_assert(kMT == 64, "K' slice: 8 lanes of 16 bytes per row, 8 rows per store");
  __shared__ __align__(16) bf16_t ks[2][kMT][KR];
  __shared__ __align__(16) bf16_t kt[8][16][TR];
  asm volatile("" ::"s"(k_raw), "s"(v_raw), "s"(P), "s"(n), "s"(d_store), "s"(T_cap), "s"(len0),
               "s"(tiles_per_wg), "s"(kp), "s"(vc));
  const int bg = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int blk = w % NB, tb0 = WPB == 1 ? 0 : w / NB;  // 8 wavefronts
  const int full = n / kMT;
  const int x0 = blockIdx.x * tiles_per_wg;
  const int x1 = min(x0 + tiles_per_wg, full);
  const bf16_t *kb = k_raw + static_cast<size_t>(bg) * n * D;
  const bf16_t *vb = v_raw + static_cast<size_t>(bg) * n * D;
  float pv[KS][8];
  load_p_raw<KS>(P, 16 * blk, pv, d_store - 1);
  // This wavefront's tokens: token blocks [TBW tb0, TBW tb0 + TBW) of each tile (all four, or
  // with two wavefronts per column block a contiguous half each), which it alone writes to its
  // slice and stores.  Store lanes: row srow + RPS j (j < NST), tokens scol .. scol + 7.
  constexpr int TBW = (kMT / 16) / WPB;   // token blocks per wavefront
  constexpr int CPR = TBW * 16 / 8;       // 16-byte chunks per slice row
  constexpr int RPS = 64 / CPR;           // slice rows per store
  constexpr int NST = 16 / RPS;           // stores per wavefront per tile
  const int srow = lane / CPR, scol = TBW * 16 * tb0 + 8 * (lane % CPR);
  bf16_t *kprow = kp + (static_cast<size_t>(bg) * d_store + min(16 * blk + srow, d_store - 1)) *
                           T_cap + len0 + scol;
  // K' row offset from store j = 0 to j = 1 (rows srow and srow + RPS, both clamped)
  const int kprow8 = (min(16 * blk + srow + RPS, d_store - 1) - min(16 * blk + srow, d_store - 1)) *
                     T_cap;
  bf16_t *vcb = vc + (static_cast<size_t>(bg) * T_cap + len0) * D;
  u32x4_t kS[kNS][CH], vS[kNS][CH];
  // this wavefront's 16 x 16 block of K' (token block tb) into its slice: lane holds dim
  // l % 16, tokens 4 (l / 16) .. + 3
  auto to_slice = [&](int tb, const f32x4_t &pr) {
    *reinterpret_cast<u32x2_t *>(&kt[w][lane & 15][16 * tb + 4 * (lane >> 4)]) =
        u32x2_t{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
  };
#define AQUA_PK_LOAD(S_, X)                                                              \
  _Pragma("unroll") for (int c = 0; c < CH; ++c) {                                       \
    const size_t off = static_cast<size_t>(X) * kMT * D + static_cast<size_t>(tid + 512 * c) * 8; \
    kS[S_][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kb + off)); \
    vS[S_][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vb + off)); \
  }
#define AQUA_PK_MFMA(BUF)                                                                \
  _Pragma("unroll") for (int tb = TBW * tb0; tb < TBW * tb0 + TBW; ++tb) {               \
    u32x4_t av[KS];                                                                      \
    _Pragma("unroll") for (int st = 0; st < KS; ++st) av[st] =                           \
        *reinterpret_cast<const u32x4_t *>(&ks[BUF][16 * tb + (lane & 15)][32 * st + 8 * (lane >> 4)]); \
    to_slice(tb, proj_mfma<KS>(av, pp));                                                 \
  }
#define AQUA_PK_TILE(S_, X, BUF)                                                         \
  {                                                                                      \
    _Pragma("unroll") for (int c = 0; c < CH; ++c) {                                     \
      const int pc = tid + 512 * c;                                                      \
      __builtin_nontemporal_store(                                                       \
          vS[S_][c], reinterpret_cast<u32x4_t *>(vcb + static_cast<size_t>(X) * kMT * D + pc * 8)); \
      *reinterpret_cast<u32x4_t *>(&ks[BUF][pc / PR][8 * (pc % PR)]) = kS[S_][c];        \
    }                                                                                    \
    lds_barrier();                                                                       \
    AQUA_PK_MFMA(BUF)                                                                    \
    bf16_t *dst = kprow + static_cast<size_t>(X) * kMT;                                  \
    _Pragma("unroll") for (int j = 0; j < NST; ++j) __builtin_nontemporal_store(         \
        *reinterpret_cast<const u32x4_t *>(&kt[w][srow + RPS * j][scol]),                \
        reinterpret_cast<u32x4_t *>(dst + j * kprow8));                                  \
  }
  // P's parts first (once per workgroup): splitting them with a tile's loads in flight would
  // need more registers than four wavefronts per SIMD leave
  PParts<KS> pp;
  split_p_parts<KS>(pv, pp);
  int tail_buf = 0;
  if (x1 - x0 >= kNS) {
    // tiles x0 .. x0 + kNS - 2 requested, then rotations of kNS tiles: each tile's loads go out
    // kNS - 1 tiles ahead of its work; the first rotation is peeled so that the loop's entry has
    // the same loads and stores in flight as its back edge (the waits inside stay exact).  Past
    // the run's end a rotation works on its last tile again, storing the same values.
#pragma unroll
    for (int s = 0; s < kNS - 1; ++s) AQUA_PK_LOAD(s, x0 + s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      AQUA_PK_LOAD((s + kNS - 1) % kNS, min(x0 + s + kNS - 1, x1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      AQUA_PK_TILE(s, x0 + s, s & 1);
    }
    for (int x = x0 + kNS; x < x1; x += kNS) {
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        AQUA_PK_LOAD((s + kNS - 1) % kNS, min(x + s + kNS - 1, x1 - 1));
        __builtin_amdgcn_sched_barrier(0);
        AQUA_PK_TILE(s, min(x + s, x1 - 1), s & 1);
      }
    }
  } else {
    // a short run: one tile at a time, LDS buffers by the run's own tile count (the tail below
    // takes the one its last tile did not use)
    for (int x = x0; x < x1; ++x) {
      AQUA_PK_LOAD(0, x);
      AQUA_PK_TILE(0, x, (x - x0) & 1);
    }
    tail_buf = (x1 - x0) & 1;
  }
  // the ragged tail (tokens full * 64 .. n - 1), by the last workgroup of the (b, g), in the LDS
  // buffer the last whole tile did not use
  const int nt = n - full * kMT;
  if (blockIdx.x != gridDim.x - 1 || nt == 0) return;
  {
    const int t0 = full * kMT;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int pc = tid + 512 * c, t = pc / PR;
      const size_t off = static_cast<size_t>(min(t0 + t, n - 1)) * D + 8 * (pc % PR);
      const u32x4_t kr = *reinterpret_cast<const u32x4_t *>(kb + off);
      const u32x4_t vr = *reinterpret_cast<const u32x4_t *>(vb + off);
      *reinterpret_cast<u32x4_t *>(&ks[tail_buf][t][8 * (pc % PR)]) = kr;
      if (t < nt)
        *reinterpret_cast<u32x4_t *>(vcb + static_cast<size_t>(t0 + t) * D + 8 * (pc % PR)) = vr;
    }
  }
  lds_barrier();
  if (tail_buf) {
    AQUA_PK_MFMA(1)
  } else {
    AQUA_PK_MFMA(0)
  }
  bf16_t *dst = kprow + static_cast<size_t>(full) * kMT;
  // each lane's 8 tokens: whole when inside the tail, else token by token up to its end
#pragma unroll
  for (int j = 0; j < NST; ++j) {
    bf16_t *d = dst + j * kprow8;
    const bf16_t *src = &kt[w][srow + RPS * j][scol];
    if (scol + 8 <= nt) {
      *reinterpret_cast<u32x4_t *>(d) = *reinterpret_cast<const u32x4_t *>(src);
    } else {
      for (int e = 0; scol + e < nt; ++e) d[e] = src[e];
    }
  }
#undef AQUA_PK_LOAD
#undef AQUA_PK_MFMA
#undef AQUA_PK_TILE
}

// Few tokens per (b, g) (a decode step's new key, an H2O slot): one workgroup of D/16 wavefronts
// per (b, g), wavefront w projecting output dims [16 w, 16 w + 16) of the n <= 16 rows.
template <int D>
__global__ __launch_bounds__(D / 16 * 64) void project_keys_small_mfma_kernel(
    const bf16_t *__restrict__ k_raw, const bf16_t *__restrict__ v_raw,
    const float *__restrict__ P, int n, int d_store, int T_cap, int len0,
    const int32_t *__restrict__ slots, bf16_t *__restrict__ kp, bf16_t *__restrict__ vc) {
  constexpr int KS = D / 32;
  __shared__ int cols[16];
  const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < n) {
    const int col = slots ? slots[static_cast<size_t>(bg) * n + tid] : len0 + tid;
    cols[tid] = (col >= 0 && col < T_cap) ? col : -1;
  }
  u32x4_t av[KS];
  load_a_row<KS>(k_raw + (static_cast<size_t>(bg) * n + min(lane & 15, n - 1)) * D, av);
  PParts<KS> pp;
  load_p_parts<KS>(P, 16 * w, pp);
  const f32x4_t x = proj_mfma<KS>(av, pp);
  __syncthreads();
  const int dim = 16 * w + (lane & 15);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int t = 4 * (lane >> 4) + rr;
    if (t < n && dim < d_store && cols[t] >= 0)
      kp[(static_cast<size_t>(bg) * d_store + dim) * T_cap + cols[t]] = f32_to_bf16_rne(x[rr]);
  }
  if (v_raw) {
    for (int e = tid; e < n * D; e += D / 16 * 64) {
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
  if constexpr (sizeof(KT) == 2) {
    const bf16_t *kr = static_cast<const bf16_t *>(k_raw);
    const bf16_t *vr = static_cast<const bf16_t *>(v_raw);
    if (n <= 16) {
      project_keys_small_mfma_kernel<D><<<dim3(B * Hkv), dim3(D / 16 * 64), 0, s>>>(
          kr, vr, P, n, d_store, T_cap, len0, slots, static_cast<bf16_t *>(kp),
          static_cast<bf16_t *>(v));
      return hipGetLastError();
    }
    const int full = n / kMT;
    if (!slots && vr && len0 % 8 == 0 && full > 0) {
      // whole tiles stream; about one workgroup per CU, each over a contiguous run of tiles (a
      // whole number of rotations where runs are long)
      const int groups = B * Hkv;
      const int per_group = std::max(1, std::min(full, (device_cu_count() + groups - 1) / groups));
      int tpw = (full + per_group - 1) / per_group;
      if (tpw >= kNS) tpw = (tpw + kNS - 1) / kNS * kNS;
      const int wgs = (full + tpw - 1) / tpw;
      project_keys_stream_kernel<D><<<dim3(wgs, groups), dim3(512), 0, s>>>(
          kr, vr, P, n, d_store, T_cap, len0, tpw, static_cast<bf16_t *>(kp),
          static_cast<bf16_t *>(v));
      return hipGetLastError();
    }
    const dim3 grid((n + kMT - 1) / kMT, B * Hkv);
    project_keys_mfma_kernel<D><<<grid, dim3(512), 0, s>>>(
        kr, vr, P, n, d_store, T_cap, len0, slots, static_cast<bf16_t *>(kp),
        static_cast<bf16_t *>(v));
    return hipGetLastError();
  } else {
    using C = ProjCfg<KT, D>;
    if (n <= kSmallN) {
      project_keys_small_kernel<KT, D><<<dim3(B * Hkv), dim3(256), 0, s>>>(
          static_cast<const KT *>(k_raw), static_cast<const KT *>(v_raw), P, n, d_store, T_cap,
          len0, slots, static_cast<KT *>(kp), static_cast<KT *>(v));
      return hipGetLastError();
    }
    const dim3 grid((n + C::TT - 1) / C::TT, B * Hkv), block(256);
    project_keys_kernel<KT, D><<<grid, block, 0, s>>>(
        static_cast<const KT *>(k_raw), static_cast<const KT *>(v_raw), P, n, d_store, T_cap,
        len0, slots, static_cast<KT *>(kp), static_cast<KT *>(v));
    return hipGetLastError();
  }
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
