/*
 * libaqua: AQUA (Attention via QUery mAgnitudes) online attention for AMD MI355X (gfx950).
 *
 * The method (arXiv 2509.11155, "AQUA: Attention via QUery mAgnitudes for Memory and Compute
 * Efficient Inference in LLMs"): an orthogonal projection P is computed offline; online, every
 * query q and key k is rotated, q' = q P and k' = k P (row vectors); each query keeps only the
 * k dimensions where |q'| is largest and computes its attention scores over those dimensions
 * only, with the usual 1/sqrt(d_head) scale, followed by a softmax and the V-weighted sum.
 * Sources: the shd-paper.top digest of the paper, section 方法详解 (技术框架), and the edgentiq
 * blog post on AQUA, section "How AQUA Works" (online step) and "AQUA-Memory" (static cut).
 *
 * Conventions shared by every call
 *  - Every call is host-side and asynchronous: it validates its arguments (before any HIP
 *    call), then enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).  It
 *    never synchronises and never allocates device memory.
 *  - All device buffers belong to the caller.  Tensors are dense row-major in the order given
 *    in brackets, with 16-byte aligned base pointers.
 *  - Errors: a non-OK status is returned and aqua_last_error() holds a thread-local message.
 *    On a validation error nothing has been enqueued.  AQUA_ERR_HIP means a launch failed.
 *  - Preconditions not checked: inputs are finite; P is orthogonal; buffers do not overlap
 *    unless stated; device buffers hold at least the sizes stated.
 *  - Calls are thread-safe; ordering between calls comes only from the stream.
 *  - Floating point: storage of K' and V is fp32 or bf16 (round to nearest even, once); all
 *    arithmetic is fp32 except the prefill contractions, which use bf16 operands (masked q' and
 *    softmax weights, rounded to nearest even) with fp32 accumulation.  Projections (q' and K')
 *    of bf16 inputs run on bf16 MFMA against an exact three-part bf16 split of the fp32 P (every
 *    product exact, fp32 accumulation) in one fixed order of operations, so a row's q' or K' is
 *    the same bits in every call that computes it; fp32 inputs are projected with fp32 fmas.
 */
#ifndef AQUA_H
#define AQUA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AQUA_OK = 0,
  AQUA_ERR_NULL = 1,      /* a required pointer is NULL */
  AQUA_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
  AQUA_ERR_DTYPE = 3,     /* unknown or unsupported dtype */
  AQUA_ERR_CAPACITY = 4,  /* the cache cannot hold the tokens asked for */
  AQUA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned */
  AQUA_ERR_WORKSPACE = 6, /* workspace missing or too small */
  AQUA_ERR_HIP = 7        /* the HIP runtime reported an error */
} aqua_status;

typedef enum { AQUA_F32 = 0, AQUA_BF16 = 1 } aqua_dtype;

/* The KV cache of one attention layer.  The memory belongs to the caller.
 *   kp: K' = K P, dimension-major [B][Hkv][d_store][T_cap]: row (b, g, i) holds projected
 *       dimension i of every cached token, so the rows of unselected dimensions are never read.
 *   v : V, token-major [B][Hkv][T_cap][d_head] (neither projected nor cut).
 *   d_store <= d_head keeps only projected dimensions 0..d_store-1 (AQUA-Memory's static cut,
 *   blog section "AQUA-Memory").  T_cap is a multiple of 64.  len (0..T_cap) is the number of
 *   valid tokens (columns 0..len-1); it is host-side metadata, advanced by aqua_project_keys in
 *   append mode.  dtype is the storage type of kp and v. */
typedef struct {
  void *kp;
  void *v;
  int32_t B, Hkv, d_head, d_store, T_cap;
  int32_t len;
  int32_t dtype; /* aqua_dtype */
} aqua_cache;

const char *aqua_version(void);
/* Message for the last non-OK status returned on this thread ("" if none). */
const char *aqua_last_error(void);

/* Online key projection (digest, 技术框架; blog, "How AQUA Works" step 2): for n new tokens per
 * (b, g), K' = K P in fp32, rounded once to c->dtype, dims 0..d_store-1 written into kp; V
 * copied into v.
 *   k_raw : device [B][Hkv][n][d_head], c->dtype.     v_raw: same shape, or NULL (V untouched).
 *   P     : device [d_head][d_head] fp32.
 *   slots : NULL = append at columns [len, len+n) and then c->len += n (AQUA_ERR_CAPACITY if
 *           len + n > T_cap); or device int32 [B][Hkv][n] destination columns, each in
 *           [0, T_cap) (not checked on the host; out-of-range entries are skipped by the kernel),
 *           and c->len is left unchanged.
 * n == 0 is a no-op. */
aqua_status aqua_project_keys(aqua_cache *c, const void *k_raw, const void *v_raw,
                              const float *P, int32_t n, const int32_t *slots, void *stream);

/* Query projection and dynamic dimension selection (digest, 核心思路 and 技术框架; blog, "How
 * AQUA Works" step 2): q' = q P in fp32, then the k dims i < d_sel with the largest |q'_i|.
 * Magnitudes are compared exactly, as the fp32 bit patterns with the sign cleared (so +0 and -0
 * tie and denormals are not flushed); equal magnitudes go to the lower index.
 *   q      : device [N][d] of dtype qdt.     P: device [d][d] fp32.    d in {64, 128}.
 *   q_proj : out device [N][d] fp32 (q'), or NULL.
 *   mask   : out device [N][d/32] uint32; bit (i % 32) of word i / 32 set iff dim i is kept;
 *            exactly k bits per row.
 *   idx    : out device [N][k] int16, the kept dims in ascending order, or NULL.
 * 1 <= k <= d_sel <= d.  N == 0 is a no-op. */
aqua_status aqua_select_dims(const void *q, int32_t qdt, int32_t N, int32_t d, const float *P,
                             int32_t d_sel, int32_t k, float *q_proj, uint32_t *mask,
                             int16_t *idx, void *stream);

/* Bytes of workspace aqua_decode needs for this cache shape and Hq query heads (any len up to
 * T_cap).  The workspace needs no initialisation and no clearing between calls, whatever it holds
 * (its cross-workgroup counters are tagged with a per-call sequence number, so the words of an
 * earlier call, of an interrupted one, of another shape, or garbage, are never taken for this
 * call's).  Calls sharing a workspace must not run concurrently (ordering on one stream is
 * enough). */
aqua_status aqua_decode_workspace(const aqua_cache *c, int32_t Hq, size_t *bytes);

/* GQA decode attention over the selected dimensions (digest, 技术框架: attention computed on
 * the selected dims only).  Query head h uses KV head h / (Hq / Hkv).  For each (b, h):
 *   s_t = scale * sum_{i selected} q'_i K'_{i,t}  for t < c->len,   p = softmax(s),
 *   out = sum_t p_t V_t.
 * Every token in [0, len) is attended (the new token is appended before the call).
 *   q_proj: device [B][Hq][d_head] fp32.      mask: device [B][Hq][d_head/32] uint32, as
 *           written by aqua_select_dims; bits of dims >= d_store are ignored.
 *   scale : usually 1/sqrt(d_head).
 *   mass  : NULL, or device fp32 [B][Hkv][T_cap]: mass[b][g][t] += sum over the group's query
 *           heads of p_t (H2O's cumulative attention; abstract and blog "Key Advantages").
 *   out   : out device [B][Hq][d_head] fp32.
 *   ws    : workspace of at least aqua_decode_workspace() bytes (see there).
 * Requires 1 <= len <= T_cap, Hq % Hkv == 0, Hq / Hkv in {1, 2, 4, 8}. */
aqua_status aqua_decode(const aqua_cache *c, int32_t Hq, const float *q_proj,
                        const uint32_t *mask, float scale, float *mass, float *out, void *ws,
                        size_t ws_bytes, void *stream);

/* One whole decode step in one launch (the online step of the digest's 技术框架 and the blog's
 * "How AQUA Works", step 2, for a token being generated): appends the new token, then every
 * query head projects its query, selects its top-k dims and attends over [0, len + 1).
 * Equivalent to aqua_project_keys(c, k_new, v_new, P, 1, NULL) + aqua_select_dims(q, ...) +
 * aqua_decode(...), fused so that no small launch sits on the critical path.
 *   q     : device [B][Hq][d_head], c->dtype (raw queries).
 *   k_new, v_new: device [B][Hkv][d_head], c->dtype (the new token's raw key and value); its K'
 *           and V are written at column len, then c->len += 1 (AQUA_ERR_CAPACITY if full).
 *   P     : device [d_head][d_head] fp32.   1 <= k <= d_sel <= d_store.
 *   mass, out, ws, ws_bytes: as aqua_decode (the same workspace size; no clearing needed).
 *   q_proj_out, mask_out: NULL, or out device [B][Hq][d_head] fp32 and [B][Hq][d_head/32]
 *           uint32 (the q' and masks used, as aqua_select_dims would write them). */
aqua_status aqua_decode_step(aqua_cache *c, int32_t Hq, const void *q, const void *k_new,
                             const void *v_new, const float *P, int32_t d_sel, int32_t k,
                             float scale, float *mass, float *out, float *q_proj_out,
                             uint32_t *mask_out, void *ws, size_t ws_bytes, void *stream);

/* aqua_decode_step without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a fixed 32 MiB device array inside the library, one per device, held until the
 * process ends.  Same arguments, results and errors as aqua_decode_step, less ws and ws_bytes;
 * AQUA_ERR_WORKSPACE if the shape needs more than 32 MiB (aqua_decode_workspace() bytes, less
 * B * Hq * T_cap * 4 when mass is NULL; e.g. B16 x Hq32 at T_cap 8448 needs 4.3 MB, 21.6 MB
 * with mass).  It allocates nothing.  Every call on a device shares that device's array, so
 * calls that may overlap on one device (different streams, threads) race: order them. */
aqua_status aqua_decode_step_noalloc(aqua_cache *c, int32_t Hq, const void *q, const void *k_new,
                                     const void *v_new, const float *P, int32_t d_sel, int32_t k,
                                     float scale, float *mass, float *out, float *q_proj_out,
                                     uint32_t *mask_out, void *stream);

/* Bytes of workspace aqua_prefill_chunk needs for a chunk of Lq queries (no clearing needed). */
aqua_status aqua_prefill_workspace(const aqua_cache *c, int32_t Hq, int32_t Lq, size_t *bytes);

/* Causal chunked prefill: the queries at positions pos0 .. pos0+Lq-1, each selecting its own
 * top-k dims (as aqua_select_dims) and attending every key at a position <= its own.  The
 * cache must already hold K' and V for [0, pos0 + Lq) (c->len >= pos0 + Lq).
 *   q     : device [B][Hq][Lq][d_head], c->dtype.     P: device [d_head][d_head] fp32.
 *   out   : out device [B][Hq][Lq][d_head] fp32.
 *   q_proj_out, mask_out: NULL, or out device [B][Hq][Lq][d_head] fp32 and
 *           [B][Hq][Lq][d_head/32] uint32 (the q' and masks used).
 *   ws    : workspace of at least aqua_prefill_workspace() bytes.
 * q' is the one aqua_select_dims computes for the same bf16 rows (bit for bit); the mask is
 * always the exact top-k of the q' written to q_proj_out.
 * Requires d_head == 128, bf16 storage, d_store % 16 == 0, T_cap <= 4194304, d_sel <= d_store,
 * Lq >= 1, pos0 >= 0. */
aqua_status aqua_prefill_chunk(const aqua_cache *c, int32_t Hq, const void *q, int32_t Lq,
                               int32_t pos0, const float *P, int32_t d_sel, int32_t k,
                               float scale, float *out, float *q_proj_out, uint32_t *mask_out,
                               void *ws, size_t ws_bytes, void *stream);

/* The starting state of an H2O compact cache (H2O combined with AQUA: abstract; blog "Key
 * Advantages"): for each (b, g), the `heavy` positions of largest mass among the positions older
 * than the recent window, [0, full->len - recent), ranked by (mass descending, position
 * ascending), in ascending position order in slots 0 .. heavy-1, then the recent positions
 * [full->len - recent, full->len) in slots heavy .. heavy+recent-1.  Each slot's K' column, V row
 * and mass are copied from the full cache.
 *   full     : the full-context cache (read only), full->len tokens.
 *   mass_full: device fp32 [B][Hkv][full->T_cap], each >= +0 (the cumulative attention so far).
 *   compact  : B, Hkv, d_head, d_store and dtype as full; T_cap == len == heavy + recent.
 *   mass     : out device fp32 [B][Hkv][heavy + recent].
 *   slot_pos : out device int32 [B][Hkv][heavy + recent] (the position each slot holds).
 * Requires heavy, recent >= 0, heavy + recent >= 1, heavy + recent <= full->len.  The buffers of
 * the compact state must not overlap the full cache. */
aqua_status aqua_h2o_init(const aqua_cache *full, const float *mass_full, int32_t heavy,
                          int32_t recent, aqua_cache *compact, float *mass, int32_t *slot_pos,
                          void *stream);

/* H2O eviction for a compact cache of n_slots slots per (b, g) (H2O combined with AQUA:
 * abstract; blog "Key Advantages").  Among the slots holding a position <= t_new - recent
 * (the non-recent ones), picks the one ranked lowest by (mass descending, position ascending),
 * i.e. least mass, latest position on ties; writes its index to victim[b][g], sets
 * slot_pos[b][g][victim] = t_new and mass[b][g][victim] = 0.  The caller then writes the new
 * token into that slot (aqua_project_keys with slots = victim).  If no slot is non-recent,
 * victim is -1 and nothing else changes.
 *   mass    : device fp32 [B][Hkv][n_slots] (read and written).
 *   slot_pos: device int32 [B][Hkv][n_slots] (read and written).
 *   victim  : out device int32 [B][Hkv].
 * All three 16-byte aligned. */
aqua_status aqua_h2o_victim(float *mass, int32_t *slot_pos, int32_t B, int32_t Hkv,
                            int32_t n_slots, int32_t t_new, int32_t recent, int32_t *victim,
                            void *stream);

/* One whole H2O decode step in one launch (H2O combined with AQUA: abstract; blog "Key
 * Advantages"; the online step of the digest's 技术框架 and the blog's "How AQUA Works" over the
 * kept tokens).  Equivalent, bit for bit, to
 *   aqua_h2o_victim(mass, slot_pos, B, Hkv, T_cap, t_new, recent, victim) +
 *   aqua_project_keys(c, k_new, v_new, P, 1, victim) +
 *   aqua_select_dims(q, ..., d_sel, k, q_proj, mask) +
 *   aqua_decode(c, Hq, q_proj, mask, scale, mass, out, ...)
 * for a compact cache whose every slot holds a token (c->len == c->T_cap <= 4096): the new
 * token at position t_new replaces the evicted slot (if any: victim is -1 when no slot is
 * older than the recent window, and then the new token is not cached), every query head selects
 * its dims and attends over all slots, and every slot's mass grows by the group's weights (the
 * replaced slot's mass restarts at 0 first).  c->len does not change.
 *   q, k_new, v_new, P, d_sel, k, scale: as aqua_decode_step (k_new/v_new [B][Hkv][d_head]).
 *   mass    : device fp32 [B][Hkv][T_cap] (read and written).
 *   slot_pos: device int32 [B][Hkv][T_cap] (read and written).
 *   victim  : out device int32 [B][Hkv].
 *   out, q_proj_out, mask_out, ws, ws_bytes: as aqua_decode_step (the same workspace size). */
aqua_status aqua_h2o_step(aqua_cache *c, int32_t Hq, const void *q, const void *k_new,
                          const void *v_new, const float *P, int32_t d_sel, int32_t k,
                          float scale, float *mass, int32_t *slot_pos, int32_t t_new,
                          int32_t recent, int32_t *victim, float *out, float *q_proj_out,
                          uint32_t *mask_out, void *ws, size_t ws_bytes, void *stream);

/* Offline projection: the Gram matrix G = X^T X of calibration vectors X, whose eigenvectors in
 * decreasing order of eigenvalue are the right singular vectors of X, i.e. the columns of P
 * (digest of arXiv 2509.11155, section 方法详解 / 技术框架: P from an SVD on a calibration
 * set; edgentiq blog, "How AQUA Works", step 1).  The d x d eigensolve is the caller's.
 *   dtype : AQUA_F32 or AQUA_BF16 (of x).
 *   x     : device [n][d], row-major, one calibration vector (a query or a key) per row.
 *   n     : rows, >= 1;  d: 64 or 128.
 *   gram  : out device double [d][d] (the full symmetric matrix).
 *   ws    : device workspace of aqua_gram_workspace() bytes (contents need no clearing).
 * Every product is exact (fp32 input as three bf16 parts each); the sums are fp32 within chunks
 * of 128 rows and fp64 across chunks, so |G - X^T X| <= gamma_m (|X|^T |X|) elementwise with
 * m = 128 (bf16) or 9 * 128 (fp32) terms, up to the fp64 sum. */
aqua_status aqua_gram_workspace(int32_t dtype, int64_t n, int32_t d, size_t *bytes);
aqua_status aqua_gram(int32_t dtype, const void *x, int64_t n, int32_t d, double *gram,
                      void *ws, size_t ws_bytes, void *stream);

/* Diagnostics.  Streaming-read probe: reads `bytes` of buf once (16-byte non-temporal loads,
 * the decode kernel's access, sixteen in flight per lane; `blocks` workgroups of 256 threads,
 * each over one contiguous slice of ceil(bytes / 16 / blocks) pieces) and writes one folded word
 * per workgroup to sink [blocks] (so that the reads are not optimised away).  Timing launches
 * gives the device's measured streaming-read bandwidth, the denominator reported next to the
 * vendor's HBM peak.  bytes a positive multiple of 16. */
aqua_status aqua_stream_read_probe(const void *buf, size_t bytes, int32_t blocks, uint32_t *sink,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQUA_H */
