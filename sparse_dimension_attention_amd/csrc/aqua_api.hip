// libaqua C ABI: argument validation (before any HIP call), workspace sizing and dispatch to the
// gfx950 kernels.  The library never allocates device memory and never synchronises.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "aqua.h"
#include "aqua_internal.h"

namespace {

thread_local char g_err[512] = "";

aqua_status fail(aqua_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

aqua_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return AQUA_OK;
  return fail(AQUA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == AQUA_BF16 ? 2 : 4; }

aqua_status check_cache(const aqua_cache *c) {
  if (!c) return fail(AQUA_ERR_NULL, "cache descriptor is NULL");
  if (!c->kp || !c->v) return fail(AQUA_ERR_NULL, "cache kp/v pointer is NULL");
  if (c->dtype != AQUA_F32 && c->dtype != AQUA_BF16)
    return fail(AQUA_ERR_DTYPE, "cache dtype %d is not AQUA_F32 or AQUA_BF16", c->dtype);
  if (c->d_head != 64 && c->d_head != 128)
    return fail(AQUA_ERR_SHAPE, "d_head %d not in {64, 128}", c->d_head);
  if (c->d_store < 1 || c->d_store > c->d_head)
    return fail(AQUA_ERR_SHAPE, "d_store %d not in [1, d_head=%d]", c->d_store, c->d_head);
  if (c->B < 1 || c->Hkv < 1) return fail(AQUA_ERR_SHAPE, "B=%d, Hkv=%d must be >= 1", c->B, c->Hkv);
  if (c->T_cap < 64 || c->T_cap % 64 != 0)
    return fail(AQUA_ERR_SHAPE, "T_cap %d must be a positive multiple of 64", c->T_cap);
  if (c->len < 0 || c->len > c->T_cap)
    return fail(AQUA_ERR_CAPACITY, "len %d not in [0, T_cap=%d]", c->len, c->T_cap);
  if (!aligned16(c->kp) || !aligned16(c->v))
    return fail(AQUA_ERR_ALIGN, "cache kp/v must be 16-byte aligned");
  return AQUA_OK;
}

aqua_status check_heads(const aqua_cache *c, int32_t Hq) {
  if (Hq < 1 || Hq % c->Hkv != 0)
    return fail(AQUA_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, c->Hkv);
  const int G = Hq / c->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(AQUA_ERR_SHAPE, "group size Hq/Hkv=%d not in {1, 2, 4, 8}", G);
  return AQUA_OK;
}

aqua_status check_prefill_cache(const aqua_cache *c, int32_t Hq) {
  if (aqua_status st = check_cache(c)) return st;
  if (aqua_status st = check_heads(c, Hq)) return st;
  if (c->dtype != AQUA_BF16) return fail(AQUA_ERR_DTYPE, "prefill needs bf16 storage");
  if (c->d_head != 128) return fail(AQUA_ERR_SHAPE, "prefill needs d_head == 128");
  if (c->d_store % 16 != 0)
    return fail(AQUA_ERR_SHAPE, "prefill needs d_store (%d) a multiple of 16", c->d_store);
  // the kernel addresses one (b, group) of K' or V with 32-bit byte offsets
  if (c->T_cap > (1 << 22))
    return fail(AQUA_ERR_SHAPE, "prefill needs T_cap (%d) <= 4194304", c->T_cap);
  return AQUA_OK;
}

// ---- the workspace of aqua_decode_step_noalloc: a file-scope device array of fixed size, one
// copy per device that runs the library, held until the process ends.  Host code never passes
// the array's name to a kernel (in host code it is a stand-in, not a device address): each
// device's address comes from hipGetSymbolAddress, called once per device with that device
// current, and is kept in scratch_ptr.  Every call on a device shares its array; nothing in it
// needs clearing (the arrival counters carry each call's epoch), and calls that overlap on one
// device race.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void *> scratch_ptr[kScratchDevices];

// This device's scratch address (nullptr with the error set if it cannot be had).
void *device_scratch(aqua_status *st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    *st = e != hipSuccess ? fail(AQUA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e))
                          : fail(AQUA_ERR_HIP, "device %d: static scratch is kept for devices "
                                 "0..%d only", dev, kScratchDevices - 1);
    return nullptr;
  }
  void *p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *st = fail(AQUA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    return nullptr;
  }
  scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// The cache and workspace fields every decode-path launch takes; S and epoch for this call.
void fill_decode_args(const aqua_cache *c, int32_t Hq, int32_t len, float scale, float *mass,
                      float *out, void *ws, aqua::DecodeArgs &a) {
  a.kp = c->kp;
  a.v = c->v;
  a.mass = mass;
  a.out = out;
  aqua::decode_workspace_carve(ws, c->dtype, c->B, Hq, c->Hkv, c->d_head, c->T_cap, a);
  a.B = c->B;
  a.Hq = Hq;
  a.Hkv = c->Hkv;
  a.d = c->d_head;
  a.d_store = c->d_store;
  a.T_cap = c->T_cap;
  a.len = len;
  a.S = aqua::decode_splits(c->dtype, Hq / c->Hkv, c->B * c->Hkv, len, aqua::device_cu_count());
  a.qscale = scale * 1.4426950408889634f;  // log2(e): scores are kept in log2 units
  a.epoch = aqua::next_epoch();
}

// aqua_decode_step once its arguments and workspace are validated
aqua_status launch_decode_step(aqua_cache *c, int32_t Hq, const void *q, const void *k_new,
                               const void *v_new, const float *P, int32_t d_sel, int32_t k,
                               float scale, float *mass, float *out, float *q_proj_out,
                               uint32_t *mask_out, void *ws, hipStream_t stream) {
  aqua::DecodeArgs a{};
  fill_decode_args(c, Hq, c->len + 1, scale, mass, out, ws, a);
  a.kp_w = c->kp;
  a.v_w = c->v;
  a.q_raw = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.P = P;
  a.q_proj_out = q_proj_out;
  a.mask_out = mask_out;
  a.d_sel = d_sel;
  a.k = k;
  if (aqua_status st =
          hip_status(aqua::launch_decode_step(c->dtype, a, stream), "aqua_decode_step launch"))
    return st;
  c->len += 1;
  return AQUA_OK;
}

}  // namespace

extern "C" {

const char *aqua_version(void) { return "libaqua 0.2.0 (gfx950)"; }

const char *aqua_last_error(void) { return g_err; }

aqua_status aqua_project_keys(aqua_cache *c, const void *k_raw, const void *v_raw,
                              const float *P, int32_t n, const int32_t *slots, void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(c)) return st;
  if (n < 0) return fail(AQUA_ERR_SHAPE, "n=%d must be >= 0", n);
  if (!k_raw || !P) return fail(AQUA_ERR_NULL, "k_raw and P are required");
  if (!aligned16(k_raw) || !aligned16(P) || (v_raw && !aligned16(v_raw)))
    return fail(AQUA_ERR_ALIGN, "k_raw, v_raw and P must be 16-byte aligned");
  if (!slots && static_cast<int64_t>(c->len) + n > c->T_cap)
    return fail(AQUA_ERR_CAPACITY, "append of n=%d at len=%d exceeds T_cap=%d", n, c->len,
                c->T_cap);
  if (n == 0) return AQUA_OK;
  hipError_t e = aqua::launch_project_keys(c->dtype, k_raw, v_raw, P, c->B, c->Hkv, n, c->d_head,
                                           c->d_store, c->T_cap, c->len, slots, c->kp, c->v,
                                           static_cast<hipStream_t>(stream));
  if (aqua_status st = hip_status(e, "aqua_project_keys launch")) return st;
  if (!slots) c->len += n;
  return AQUA_OK;
}

aqua_status aqua_select_dims(const void *q, int32_t qdt, int32_t N, int32_t d, const float *P,
                             int32_t d_sel, int32_t k, float *q_proj, uint32_t *mask,
                             int16_t *idx, void *stream) {
  g_err[0] = 0;
  if (!q || !P || !mask) return fail(AQUA_ERR_NULL, "q, P and mask are required");
  if (qdt != AQUA_F32 && qdt != AQUA_BF16)
    return fail(AQUA_ERR_DTYPE, "q dtype %d is not AQUA_F32 or AQUA_BF16", qdt);
  if (d != 64 && d != 128) return fail(AQUA_ERR_SHAPE, "d %d not in {64, 128}", d);
  if (N < 0) return fail(AQUA_ERR_SHAPE, "N=%d must be >= 0", N);
  if (!(1 <= k && k <= d_sel && d_sel <= d))
    return fail(AQUA_ERR_SHAPE, "need 1 <= k (%d) <= d_sel (%d) <= d (%d)", k, d_sel, d);
  if (!aligned16(q) || !aligned16(P) || !aligned16(mask) || (q_proj && !aligned16(q_proj)))
    return fail(AQUA_ERR_ALIGN, "q, P, mask and q_proj must be 16-byte aligned");
  if (N == 0) return AQUA_OK;
  return hip_status(aqua::launch_select(q, qdt, N, d, P, d_sel, k, q_proj, mask, idx,
                                        static_cast<hipStream_t>(stream)),
                    "aqua_select_dims launch");
}

aqua_status aqua_decode_workspace(const aqua_cache *c, int32_t Hq, size_t *bytes) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(c)) return st;
  if (aqua_status st = check_heads(c, Hq)) return st;
  if (!bytes) return fail(AQUA_ERR_NULL, "bytes is NULL");
  *bytes = aqua::decode_workspace_bytes(c->dtype, c->B, Hq, c->Hkv, c->d_head, c->T_cap);
  return AQUA_OK;
}

aqua_status aqua_decode(const aqua_cache *c, int32_t Hq, const float *q_proj,
                        const uint32_t *mask, float scale, float *mass, float *out, void *ws,
                        size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(c)) return st;
  if (aqua_status st = check_heads(c, Hq)) return st;
  if (!q_proj || !mask || !out) return fail(AQUA_ERR_NULL, "q_proj, mask and out are required");
  if (!ws) return fail(AQUA_ERR_WORKSPACE, "workspace is NULL");
  if (c->len < 1) return fail(AQUA_ERR_SHAPE, "len=%d: decode needs at least one token", c->len);
  if (!aligned16(q_proj) || !aligned16(mask) || !aligned16(out) || !aligned16(ws) ||
      (mass && !aligned16(mass)))
    return fail(AQUA_ERR_ALIGN, "q_proj, mask, out, mass and ws must be 16-byte aligned");
  const size_t need =
      aqua::decode_workspace_bytes(c->dtype, c->B, Hq, c->Hkv, c->d_head, c->T_cap);
  if (ws_bytes < need)
    return fail(AQUA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);

  aqua::DecodeArgs a{};
  fill_decode_args(c, Hq, c->len, scale, mass, out, ws, a);
  a.q_proj = q_proj;
  a.mask = mask;
  return hip_status(aqua::launch_decode(c->dtype, a, static_cast<hipStream_t>(stream)),
                    "aqua_decode launch");
}

aqua_status aqua_decode_step(aqua_cache *c, int32_t Hq, const void *q, const void *k_new,
                             const void *v_new, const float *P, int32_t d_sel, int32_t k,
                             float scale, float *mass, float *out, float *q_proj_out,
                             uint32_t *mask_out, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(c)) return st;
  if (aqua_status st = check_heads(c, Hq)) return st;
  if (!q || !k_new || !v_new || !P || !out)
    return fail(AQUA_ERR_NULL, "q, k_new, v_new, P and out are required");
  if (!ws) return fail(AQUA_ERR_WORKSPACE, "workspace is NULL");
  if (!(1 <= k && k <= d_sel && d_sel <= c->d_store))
    return fail(AQUA_ERR_SHAPE, "need 1 <= k (%d) <= d_sel (%d) <= d_store (%d)", k, d_sel,
                c->d_store);
  if (static_cast<int64_t>(c->len) + 1 > c->T_cap)
    return fail(AQUA_ERR_CAPACITY, "append at len=%d exceeds T_cap=%d", c->len, c->T_cap);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(P) ||
      !aligned16(out) || !aligned16(ws) || (mass && !aligned16(mass)) ||
      (q_proj_out && !aligned16(q_proj_out)) || (mask_out && !aligned16(mask_out)))
    return fail(AQUA_ERR_ALIGN, "all buffers must be 16-byte aligned");
  const size_t need =
      aqua::decode_workspace_bytes(c->dtype, c->B, Hq, c->Hkv, c->d_head, c->T_cap);
  if (ws_bytes < need)
    return fail(AQUA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return launch_decode_step(c, Hq, q, k_new, v_new, P, d_sel, k, scale, mass, out, q_proj_out,
                            mask_out, ws, static_cast<hipStream_t>(stream));
}


aqua_status aqua_decode_step_noalloc(aqua_cache *c, int32_t Hq, const void *q,
                                     const void *k_new, const void *v_new, const float *P,
                                     int32_t d_sel, int32_t k, float scale, float *mass,
                                     float *out, float *q_proj_out, uint32_t *mask_out,
                                     void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(c)) return st;
  if (aqua_status st = check_heads(c, Hq)) return st;
  if (!q || !k_new || !v_new || !P || !out)
    return fail(AQUA_ERR_NULL, "q, k_new, v_new, P and out are required");
  if (!(1 <= k && k <= d_sel && d_sel <= c->d_store))
    return fail(AQUA_ERR_SHAPE, "need 1 <= k (%d) <= d_sel (%d) <= d_store (%d)", k, d_sel,
                c->d_store);
  if (static_cast<int64_t>(c->len) + 1 > c->T_cap)
    return fail(AQUA_ERR_CAPACITY, "append at len=%d exceeds T_cap=%d", c->len, c->T_cap);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(P) ||
      !aligned16(out) || (mass && !aligned16(mass)) || (q_proj_out && !aligned16(q_proj_out)) ||
      (mask_out && !aligned16(mask_out)))
    return fail(AQUA_ERR_ALIGN, "all buffers must be 16-byte aligned");
  // the workspace layout of aqua_decode_step; its last region (scores) only in mass mode
  size_t need = aqua::decode_workspace_bytes(c->dtype, c->B, Hq, c->Hkv, c->d_head, c->T_cap);
  if (!mass) need -= static_cast<size_t>(c->B) * Hq * c->T_cap * 4;
  if (need > kScratchBytes)
    return fail(AQUA_ERR_WORKSPACE, "this shape needs %zu bytes of workspace; the static scratch "
                "of aqua_decode_step_noalloc holds %zu (use aqua_decode_step with a workspace)",
                need, kScratchBytes);
  aqua_status st = AQUA_OK;
  void *ws = device_scratch(&st);
  if (!ws) return st;
  return launch_decode_step(c, Hq, q, k_new, v_new, P, d_sel, k, scale, mass, out, q_proj_out,
                            mask_out, ws, static_cast<hipStream_t>(stream));
}

aqua_status aqua_prefill_workspace(const aqua_cache *c, int32_t Hq, int32_t Lq, size_t *bytes) {
  g_err[0] = 0;
  if (aqua_status st = check_prefill_cache(c, Hq)) return st;
  if (!bytes) return fail(AQUA_ERR_NULL, "bytes is NULL");
  if (Lq < 1) return fail(AQUA_ERR_SHAPE, "Lq=%d must be >= 1", Lq);
  *bytes = aqua::prefill_workspace_bytes(c->B, Hq, Lq);
  return AQUA_OK;
}

aqua_status aqua_prefill_chunk(const aqua_cache *c, int32_t Hq, const void *q, int32_t Lq,
                               int32_t pos0, const float *P, int32_t d_sel, int32_t k,
                               float scale, float *out, float *q_proj_out, uint32_t *mask_out,
                               void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_prefill_cache(c, Hq)) return st;
  if (!q || !P || !out) return fail(AQUA_ERR_NULL, "q, P and out are required");
  if (!ws) return fail(AQUA_ERR_WORKSPACE, "workspace is NULL");
  if (Lq < 1 || pos0 < 0) return fail(AQUA_ERR_SHAPE, "Lq=%d >= 1 and pos0=%d >= 0 needed", Lq, pos0);
  if (static_cast<int64_t>(pos0) + Lq > c->len)
    return fail(AQUA_ERR_CAPACITY, "pos0 + Lq = %lld exceeds the cached len %d",
                static_cast<long long>(pos0) + Lq, c->len);
  if (!(1 <= k && k <= d_sel && d_sel <= c->d_store))
    return fail(AQUA_ERR_SHAPE, "need 1 <= k (%d) <= d_sel (%d) <= d_store (%d)", k, d_sel,
                c->d_store);
  if (!aligned16(q) || !aligned16(P) || !aligned16(out) || !aligned16(ws) ||
      (q_proj_out && !aligned16(q_proj_out)) || (mask_out && !aligned16(mask_out)))
    return fail(AQUA_ERR_ALIGN, "all buffers must be 16-byte aligned");
  const size_t need = aqua::prefill_workspace_bytes(c->B, Hq, Lq);
  if (ws_bytes < need)
    return fail(AQUA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return hip_status(aqua::launch_prefill(c->kp, c->v, c->B, Hq, c->Hkv, c->d_store, c->T_cap, q,
                                         Lq, pos0, P, d_sel, k, scale, out, q_proj_out,
                                         mask_out, ws, static_cast<hipStream_t>(stream)),
                    "aqua_prefill_chunk launch");
}

aqua_status aqua_h2o_victim(float *mass, int32_t *slot_pos, int32_t B, int32_t Hkv,
                            int32_t n_slots, int32_t t_new, int32_t recent, int32_t *victim,
                            void *stream) {
  g_err[0] = 0;
  if (!mass || !slot_pos || !victim) return fail(AQUA_ERR_NULL, "mass, slot_pos, victim required");
  if (B < 1 || Hkv < 1 || n_slots < 1)
    return fail(AQUA_ERR_SHAPE, "B=%d, Hkv=%d, n_slots=%d must be >= 1", B, Hkv, n_slots);
  if (recent < 0 || t_new < 0)
    return fail(AQUA_ERR_SHAPE, "t_new=%d and recent=%d must be >= 0", t_new, recent);
  if (!aligned16(mass) || !aligned16(slot_pos) || !aligned16(victim))
    return fail(AQUA_ERR_ALIGN, "mass, slot_pos and victim must be 16-byte aligned");
  return hip_status(aqua::launch_h2o_victim(mass, slot_pos, B, Hkv, n_slots, t_new, recent,
                                            victim, static_cast<hipStream_t>(stream)),
                    "aqua_h2o_victim launch");
}

aqua_status aqua_h2o_step(aqua_cache *c, int32_t Hq, const void *q, const void *k_new,
                          const void *v_new, const float *P, int32_t d_sel, int32_t k,
                          float scale, float *mass, int32_t *slot_pos, int32_t t_new,
                          int32_t recent, int32_t *victim, float *out, float *q_proj_out,
                          uint32_t *mask_out, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(c)) return st;
  if (aqua_status st = check_heads(c, Hq)) return st;
  if (!q || !k_new || !v_new || !P || !mass || !slot_pos || !victim || !out)
    return fail(AQUA_ERR_NULL, "q, k_new, v_new, P, mass, slot_pos, victim and out are required");
  if (!ws) return fail(AQUA_ERR_WORKSPACE, "workspace is NULL");
  if (c->len != c->T_cap)
    return fail(AQUA_ERR_SHAPE, "len=%d: every slot of the compact cache must hold a token "
                "(len == T_cap=%d)", c->len, c->T_cap);
  if (c->len > aqua::kDecodeShortMax)
    return fail(AQUA_ERR_SHAPE, "%d slots: the fused H2O step takes at most %d", c->len,
                aqua::kDecodeShortMax);
  if (!(1 <= k && k <= d_sel && d_sel <= c->d_store))
    return fail(AQUA_ERR_SHAPE, "need 1 <= k (%d) <= d_sel (%d) <= d_store (%d)", k, d_sel,
                c->d_store);
  if (t_new < 0 || recent < 0)
    return fail(AQUA_ERR_SHAPE, "t_new=%d and recent=%d must be >= 0", t_new, recent);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(P) ||
      !aligned16(out) || !aligned16(ws) || !aligned16(mass) ||
      (q_proj_out && !aligned16(q_proj_out)) || (mask_out && !aligned16(mask_out)))
    return fail(AQUA_ERR_ALIGN, "all buffers must be 16-byte aligned");
  const size_t need =
      aqua::decode_workspace_bytes(c->dtype, c->B, Hq, c->Hkv, c->d_head, c->T_cap);
  if (ws_bytes < need)
    return fail(AQUA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);

  aqua::DecodeArgs a{};
  fill_decode_args(c, Hq, c->len, scale, mass, out, ws, a);
  a.S = (c->len + aqua::kShortChunk - 1) / aqua::kShortChunk;  // the step runs the short kernel
  a.kp_w = c->kp;
  a.v_w = c->v;
  a.q_raw = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.P = P;
  a.q_proj_out = q_proj_out;
  a.mask_out = mask_out;
  a.d_sel = d_sel;
  a.k = k;
  aqua::H2OArgs h{};
  h.slot_pos = slot_pos;
  h.victim = victim;
  h.t_new = t_new;
  h.recent = recent;
  return hip_status(aqua::launch_h2o_step(c->dtype, a, h, static_cast<hipStream_t>(stream)),
                    "aqua_h2o_step launch");
}

aqua_status aqua_h2o_init(const aqua_cache *full, const float *mass_full, int32_t heavy,
                          int32_t recent, aqua_cache *compact, float *mass, int32_t *slot_pos,
                          void *stream) {
  g_err[0] = 0;
  if (aqua_status st = check_cache(full)) return st;
  if (aqua_status st = check_cache(compact)) return st;
  if (!mass_full || !mass || !slot_pos)
    return fail(AQUA_ERR_NULL, "mass_full, mass and slot_pos are required");
  if (compact->B != full->B || compact->Hkv != full->Hkv || compact->d_head != full->d_head ||
      compact->d_store != full->d_store || compact->dtype != full->dtype)
    return fail(AQUA_ERR_SHAPE, "the compact cache must have the full cache's B, Hkv, d_head, "
                "d_store and dtype");
  if (heavy < 0 || recent < 0 || static_cast<int64_t>(heavy) + recent < 1)
    return fail(AQUA_ERR_SHAPE, "heavy=%d and recent=%d must be >= 0 with a positive sum", heavy,
                recent);
  if (compact->T_cap != heavy + recent || compact->len != compact->T_cap)
    return fail(AQUA_ERR_SHAPE, "the compact cache needs T_cap == len == heavy + recent = %d "
                "(T_cap=%d, len=%d)", heavy + recent, compact->T_cap, compact->len);
  if (static_cast<int64_t>(heavy) + recent > full->len)
    return fail(AQUA_ERR_CAPACITY, "heavy + recent = %d exceeds the cached len %d",
                heavy + recent, full->len);
  if (!aligned16(mass_full) || !aligned16(mass) || !aligned16(slot_pos))
    return fail(AQUA_ERR_ALIGN, "mass_full, mass and slot_pos must be 16-byte aligned");
  return hip_status(aqua::launch_h2o_init(full->dtype, full->kp, full->v, mass_full, full->B,
                                          full->Hkv, full->d_head, full->d_store, full->T_cap,
                                          full->len, heavy, recent, compact->kp, compact->v,
                                          mass, slot_pos, static_cast<hipStream_t>(stream)),
                    "aqua_h2o_init launch");
}

static aqua_status gram_check(int32_t dtype, int64_t n, int32_t d) {
  if (dtype != AQUA_F32 && dtype != AQUA_BF16) return fail(AQUA_ERR_DTYPE, "dtype %d", dtype);
  if (d != 64 && d != 128) return fail(AQUA_ERR_SHAPE, "d=%d must be 64 or 128", d);
  if (n < 1 || n > (static_cast<int64_t>(1) << 40) / d)
    return fail(AQUA_ERR_SHAPE, "n=%lld out of range", static_cast<long long>(n));
  return AQUA_OK;
}

aqua_status aqua_gram_workspace(int32_t dtype, int64_t n, int32_t d, size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(AQUA_ERR_NULL, "bytes is required");
  const aqua_status st = gram_check(dtype, n, d);
  if (st != AQUA_OK) return st;
  *bytes = aqua::gram_workspace_bytes(n, d);
  return AQUA_OK;
}

aqua_status aqua_gram(int32_t dtype, const void *x, int64_t n, int32_t d, double *gram,
                      void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  const aqua_status st = gram_check(dtype, n, d);
  if (st != AQUA_OK) return st;
  if (!x || !gram || !ws) return fail(AQUA_ERR_NULL, "x, gram and ws are required");
  if (!aligned16(x) || !aligned16(gram) || !aligned16(ws))
    return fail(AQUA_ERR_ALIGN, "x, gram and ws must be 16-byte aligned");
  const size_t need = aqua::gram_workspace_bytes(n, d);
  if (ws_bytes < need)
    return fail(AQUA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  return hip_status(aqua::launch_gram(dtype, x, n, d, gram, ws, static_cast<hipStream_t>(stream)),
                    "aqua_gram launch");
}

aqua_status aqua_stream_read_probe(const void *buf, size_t bytes, int32_t blocks,
                                   uint32_t *sink, void *stream) {
  g_err[0] = 0;
  if (!buf || !sink) return fail(AQUA_ERR_NULL, "buf and sink are required");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(AQUA_ERR_SHAPE, "bytes (%zu) must be a positive multiple of 16", bytes);
  if (blocks < 1) return fail(AQUA_ERR_SHAPE, "blocks=%d must be >= 1", blocks);
  if (!aligned16(buf) || !aligned16(sink))
    return fail(AQUA_ERR_ALIGN, "buf and sink must be 16-byte aligned");
  return hip_status(aqua::launch_stream_read(buf, bytes, blocks, sink,
                                             static_cast<hipStream_t>(stream)),
                    "aqua_stream_read_probe launch");
}

}  // extern "C"
