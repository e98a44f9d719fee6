// Host side of the decode path: launch geometry, workspace layout and dispatch to the kernels
// (decode_kernels.h, instantiated in decode_split_*.hip, decode_step_bf16.hip and
// decode_short_*.hip).
#include <atomic>

#include "aqua_internal.h"

namespace aqua {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not read yet
std::atomic<uint32_t> g_epoch{0};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

uint32_t next_epoch() {
  uint32_t e;
  do e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  while (e == 0);
  return e;
}

// Workgroups of 4 wavefronts, each wavefront owning 64 lanes x 16 bytes of tokens (for G = 8,
// whose LDS numerators are twice as large per wavefront, 2-wavefront workgroups ran the 16 x
// 8-group, 8192-token fused step in 154 us against 103 with 4: LDS held only three of them per
// CU).  For G = 4 and G = 8, 8 wavefronts per
// workgroup when the full 8-wavefront splits alone give every CU a workgroup: one 512-thread
// workgroup per CU, whose wavefronts are all of one age (with two 4-wavefront workgroups per CU
// the second one resident ran ~4 us behind the first; 8 measured 1 us faster on the 16 x 8-group,
// 8192-token decode).  Counting only full splits keeps the finer layout where a ragged last split
// would leave CUs without work (at 16 x 8 groups and 4097 .. 8191 tokens, 128 workgroups of 4096
// tokens carry nearly all of it), and where the grid is small (a 32-workgroup grid at 16384 tokens
// and batch 1 ran 48 against 35 us).  The 8-wavefront grid must also end on a (nearly) whole round
// of one workgroup per CU: a part-filled last round runs after the first one, where the
// 4-wavefront grid (two per CU) packs its splits more finely.  Measured at 16 x 8 groups (decode
// kernel): 8193 .. 12288 tokens, 384 8-wavefront workgroups (1.5 rounds): 117 .. 138 us against
// 101 .. 130 us with 4 wavefronts; 12289 .. 16384 tokens, 512 (2 rounds): 136 .. 166 us against
// 144 .. 184 us.
DecodeLayout decode_layout(int dtype, int G, int groups, int len, int cus) {
  DecodeLayout L;
  L.tokens_wave = 64 * (dtype == 1 ? 8 : 4);
  L.waves = 4;
  if ((G == 4 || G == 8) && groups > 0) {
    const long wide = 8L * L.tokens_wave;
    const long full_wide = static_cast<long>(len) / wide;
    const long wgs = static_cast<long>(groups) * ((len + wide - 1) / wide);
    const long last_round = wgs % cus;  // workgroups in a part-filled last round, if any
    const bool whole_rounds = last_round == 0 || 4 * last_round >= 3L * cus;
    if (static_cast<long>(groups) * full_wide >= cus && whole_rounds) L.waves = 8;
  }
  L.split = L.waves * L.tokens_wave;
  return L;
}

// The short kernel (256-token workgroups; its fused form one workgroup per CU at a time) for up
// to kDecodeShortMax tokens while its grid fills at most two rounds of the device; past that the
// split-T kernel, whose floor is one 512-token segment per wavefront (~34 us for the decode,
// ~39 us for the fused step), is faster.  Measured, fused step / decode, short against split-T
// (Hq 32, Hkv 8, d 128, k 96): B4 x 4096 tokens (512 short workgroups) 39.3 / 23.5 against
// 39.5 / 34.1 us; B8 x 4096 and B16 x 2048 (1024) 75.0 / 41.0 against 39.5 / 34.3 us; B16 x 4096
// (2048) 142.8 / 71.7 against 49.8 / 44.9 us; B1 x 256 18.7 / 12.7 against 32.1 / 26.9 us.
bool decode_short(int len, int groups, int cus) {
  return len <= kDecodeShortMax &&
         static_cast<long>(groups) * ((len + kShortChunk - 1) / kShortChunk) <= 2L * cus;
}

int decode_splits(int dtype, int G, int groups, int len, int cus) {
  if (decode_short(len, groups, cus)) return (len + kShortChunk - 1) / kShortChunk;
  const DecodeLayout L = decode_layout(dtype, G, groups, len, cus);
  return (len + L.split - 1) / L.split;
}

namespace {
// partials per head: enough for any len <= T_cap in either layout
size_t partial_slots(int dtype, int G, int T_cap) {
  const DecodeLayout L = decode_layout(dtype, G, 0, T_cap, 1);  // the finest layout: most splits
  const size_t s_long = (static_cast<size_t>(T_cap) + L.split - 1) / L.split;
  const int short_len = T_cap < kDecodeShortMax ? T_cap : kDecodeShortMax;
  const size_t s_short = (static_cast<size_t>(short_len) + kShortChunk - 1) / kShortChunk;
  return s_long > s_short ? s_long : s_short;
}
}  // namespace

// Workspace: an arrival counter per (b, g), one per run of kMergeFan splits of each (b, g), the
// partials, then the scores (mass mode).  Nothing in it needs clearing: the counters carry the
// epoch of the call that wrote them (arrive_last), and partials and scores are written before
// they are read.
size_t decode_workspace_bytes(int dtype, int B, int Hq, int Hkv, int d, int T_cap) {
  const size_t S = partial_slots(dtype, Hq / Hkv, T_cap);
  const size_t runs = (S + kMergeFan - 1) / kMergeFan;
  return align256(static_cast<size_t>(B) * Hkv * 8) +
         align256(static_cast<size_t>(B) * Hkv * runs * 8) +
         align256(static_cast<size_t>(B) * Hq * S * (d + 2) * 4) +
         static_cast<size_t>(B) * Hq * T_cap * 4;
}

void decode_workspace_carve(void *ws, int dtype, int B, int Hq, int Hkv, int d, int T_cap,
                            DecodeArgs &a) {
  const size_t S = partial_slots(dtype, Hq / Hkv, T_cap);
  const size_t runs = (S + kMergeFan - 1) / kMergeFan;
  char *p = static_cast<char *>(ws);
  a.counters = reinterpret_cast<uint64_t *>(p);
  p += align256(static_cast<size_t>(B) * Hkv * 8);
  a.run_counters = reinterpret_cast<uint64_t *>(p);
  a.run_stride = static_cast<int>(runs);
  p += align256(static_cast<size_t>(B) * Hkv * runs * 8);
  a.partials = reinterpret_cast<float *>(p);
  p += align256(static_cast<size_t>(B) * Hq * S * (d + 2) * 4);
  a.scores = reinterpret_cast<float *>(p);
}

namespace {
hipError_t launch_split(int dtype, const DecodeArgs &a0, bool fused, hipStream_t s) {
  const int cus = device_cu_count();
  const DecodeLayout L = decode_layout(dtype, a0.Hq / a0.Hkv, a0.B * a0.Hkv, a0.len, cus);
  // Two waves per SIMD stay resident: 8 / waves workgroups per CU.  The ragged last split of
  // each group is dealt last where the grid takes more than one round (decode_kernel).
  DecodeArgs a = a0;
  const long slots = static_cast<long>(cus) * (8 / L.waves);
  a.tail_last = (a.S >= 2 && a.len % L.split != 0 &&
                 static_cast<long>(a.S) * a.B * a.Hkv > slots) ? 1 : 0;
  if (dtype == 1) return fused ? launch_split_step_bf16(a, L, s) : launch_split_bf16(a, L, s);
  return launch_split_f32(a, L, fused, s);
}

hipError_t launch_short(int dtype, const DecodeArgs &a, const H2OArgs &h, int mode,
                        hipStream_t s) {
  return dtype == 1 ? launch_short_bf16(a, h, mode, s) : launch_short_f32(a, h, mode, s);
}
}  // namespace

hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s) {
  if (decode_short(a.len, a.B * a.Hkv, device_cu_count()))
    return launch_short(dtype, a, H2OArgs{}, kShortPlain, s);
  return launch_split(dtype, a, false, s);
}

// a.S must be decode_splits(dtype, G, B * Hkv, a.len, cus): the short kernel's chunk count where
// decode_short holds
hipError_t launch_decode_step(int dtype, const DecodeArgs &a, hipStream_t s) {
  if (decode_short(a.len, a.B * a.Hkv, device_cu_count()))
    return launch_short(dtype, a, H2OArgs{}, kShortStep, s);
  return launch_split(dtype, a, true, s);
}

hipError_t launch_h2o_step(int dtype, const DecodeArgs &a, const H2OArgs &h, hipStream_t s) {
  return launch_short(dtype, a, h, kShortH2O, s);
}

}  // namespace aqua
