"""Plain fp64 CPU oracle of AQUA's online attention step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module; only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
It shares no code with the HIP library and never calls it.

Sources (the method is described in prose only; no formula or listing is printed):
  [abs]    "AQUA: Attention via QUery mAgnitudes for Memory and Compute Efficient Inference in
           LLMs", arXiv 2509.11155, abstract (English original on the shd-paper.top digest).
  [frame]  the same digest page, section "方法详解", paragraph "技术框架" (technical framework):
           project q and k with the offline matrix, keep the dimensions where the projected
           query is largest in magnitude, compute attention only on those dimensions.
  [how]    the edgentiq blog post on AQUA, section "How AQUA Works", step 2 (online inference).
  [mem]    the same blog post, section "AQUA-Memory" (static dimension cut before caching, then
           dynamic selection within the kept dimensions).
  [h2o]    [abs] and the blog's "Key Advantages" (AQUA combined with H2O token eviction).
  [off]    [frame] (the offline phase: a projection learned by SVD on a calibration set) and the
           blog's "How AQUA Works", step 1 (offline projection computation).

Where the pages leave a step open, the reading taken is stated at the function.  Every
function works in float64 on exactly the values it is given; callers pass the stored
(rounded) input values.

Pins: every function here is pinned by tests that do not re-type its formula (closed forms,
library routines, brute force, invariants).  None is "parity unpinned" except the pages' own
quality claims, which this oracle does not model.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to_storage", "project", "project_keys_stored", "select", "sparse_scores", "softmax",
    "attend", "decode", "prefill", "chunked_prefill", "split_partials", "combine_partials",
    "h2o_seed_mass", "h2o_heavy_set", "h2o_step", "h2o_run", "calibrate",
]


# ----------------------------------------------------------------------------------------------
# Storage formats.  The pages fix no precision; the cache stores K' and V in the storage dtype
# of the workload (fp32 or bf16), rounded once, to nearest with ties to even.
# ----------------------------------------------------------------------------------------------
def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Nearest value representable in `dtype` ('f64', 'f32', 'bf16'), ties to even, as fp64.

    bf16 keeps fp32's exponent range and 8 significant bits: a finite x = m * 2^e with
    0.5 <= |m| < 1 is rounded on the grid 2^(e-8); below the smallest normal (2^-126) the grid
    stays at 2^-133.  np.round rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        _, e = np.frexp(x)
        quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
        return np.round(x / quantum) * quantum
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------------------------------------
# Online projection: q' = q P and K' = K P with row vectors [frame], [how].
# ----------------------------------------------------------------------------------------------
def project(x: np.ndarray, P: np.ndarray) -> np.ndarray:
    """x' = x P for row vectors x (any leading shape), P [d][d]."""
    return np.asarray(x, np.float64) @ np.asarray(P, np.float64)


def project_keys_stored(K: np.ndarray, P: np.ndarray, dtype: str, d_store: int) -> np.ndarray:
    """The cached K': K P rounded once to the storage dtype, keeping dims 0..d_store-1 [mem]."""
    return round_to_storage(project(K, P), dtype)[..., :d_store]


# ----------------------------------------------------------------------------------------------
# Dynamic dimension selection [frame], [how]: keep the k dims with the largest |q'_i| among
# the d_sel eligible ones.  Ties (equal magnitude, including +0/-0) go to the lower index
# (a reading: the pages are silent on ties).
# ----------------------------------------------------------------------------------------------
def select(qp: np.ndarray, d_sel: int, k: int) -> np.ndarray:
    """Boolean mask [..., d] with exactly k ones per row, all among dims < d_sel."""
    qp = np.asarray(qp, np.float64)
    d = qp.shape[-1]
    if not (1 <= k <= d_sel <= d):
        raise ValueError("need 1 <= k <= d_sel <= d")
    if not np.all(np.isfinite(qp)):
        raise ValueError("q' must be finite")
    rows = qp.reshape(-1, d)
    mask = np.zeros(rows.shape, dtype=bool)
    for r in range(rows.shape[0]):
        mag = np.abs(rows[r, :d_sel])
        order = np.argsort(-mag, kind="stable")  # magnitude descending, index ascending on ties
        mask[r, order[:k]] = True
    return mask.reshape(qp.shape)


# ----------------------------------------------------------------------------------------------
# Scores over the selected dims only [frame], [how]; the usual 1/sqrt(d_head) scale for every k
# (a reading: no compensation for the dropped dims).  Softmax and the V-weighted sum are the
# standard ones; V is neither projected nor truncated.
# ----------------------------------------------------------------------------------------------
def sparse_scores(qp_row: np.ndarray, mask_row: np.ndarray, Kp: np.ndarray,
                  scale: float) -> np.ndarray:
    """s_t = scale * sum_{i in S} q'_i K'_{t,i} for every row t of Kp [T][d_store]."""
    sel = np.nonzero(mask_row)[0]
    if sel.size and sel.max() >= Kp.shape[-1]:
        raise ValueError("a selected dimension is not stored")
    return (Kp[:, sel] @ qp_row[sel]) * float(scale)


def softmax(s: np.ndarray) -> np.ndarray:
    z = np.exp(s - np.max(s))
    return z / np.sum(z)


def attend(qp_row, mask_row, Kp, V, scale):
    """(output row [dv], probabilities [T]) of one query over the rows of Kp/V."""
    p = softmax(sparse_scores(qp_row, mask_row, Kp, scale))
    return p @ V, p


def decode(qp, mask, Kp, V, scale, length=None, return_p=False):
    """GQA decode.  qp, mask [B][Hq][d]; Kp [B][Hkv][T][d_store] (token-major here);
    V [B][Hkv][T][dv].  Query head h reads KV head floor(h / G), G = Hq / Hkv (contiguous
    groups; a reading).  Attends tokens [0, length) (default all T)."""
    B, Hq, _ = qp.shape
    Hkv = Kp.shape[1]
    G = Hq // Hkv
    T = Kp.shape[2] if length is None else int(length)
    out = np.zeros((B, Hq, V.shape[-1]))
    ps = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            out[b, h], ps[b, h] = attend(qp[b, h], mask[b, h], Kp[b, g, :T], V[b, g, :T], scale)
    return (out, ps) if return_p else out


def prefill(qp, mask, Kp, V, positions, scale):
    """Causal attention for query rows at `positions` [L]: row i attends keys t <= positions[i]
    (inclusive; a reading).  qp, mask [B][Hq][L][d]; Kp [B][Hkv][T][d_store]; V [B][Hkv][T][dv]."""
    B, Hq, L, _ = qp.shape
    Hkv = Kp.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, L, V.shape[-1]))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(L):
                n = int(positions[i]) + 1
                out[b, h, i], _ = attend(qp[b, h, i], mask[b, h, i], Kp[b, g, :n], V[b, g, :n],
                                         scale)
    return out


def chunked_prefill(q, K, V, P, d_sel, k, scale, chunk, kv_dtype="f64", d_store=None):
    """The chunked schedule: for each chunk of `chunk` positions, append the chunk's K' (and V)
    to the cache, then let each of the chunk's queries select its own dims and attend causally.
    q [B][Hq][T][d], K, V [B][Hkv][T][d] raw stored values."""
    B, Hq, T, d = q.shape
    ds = d if d_store is None else d_store
    Kp = np.zeros((K.shape[0], K.shape[1], 0, ds))
    Vc = np.zeros((V.shape[0], V.shape[1], 0, V.shape[-1]))
    out = np.zeros((B, Hq, T, V.shape[-1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        Kp = np.concatenate([Kp, project_keys_stored(K[:, :, c0:c1], P, kv_dtype, ds)], axis=2)
        Vc = np.concatenate([Vc, np.asarray(V[:, :, c0:c1], np.float64)], axis=2)
        qp = project(q[:, :, c0:c1], P)
        m = select(qp, d_sel, k)
        out[:, :, c0:c1] = prefill(qp, m, Kp, Vc, np.arange(c0, c1), scale)
    return out


# ----------------------------------------------------------------------------------------------
# Split-T partials and their combination (the flash-decoding style final reduction).
# Partial j over token set T_j: m_j = max s, l_j = sum e^(s - m_j), o_j = sum e^(s - m_j) V.
# Combined: M = max m_j, L = sum e^(m_j - M) l_j, o = sum e^(m_j - M) o_j / L.
# ----------------------------------------------------------------------------------------------
def split_partials(s: np.ndarray, V: np.ndarray, bounds):
    parts = []
    for a, b in bounds:
        sj = s[a:b]
        m = np.max(sj)
        e = np.exp(sj - m)
        parts.append((m, np.sum(e), e @ V[a:b]))
    return parts


def combine_partials(parts):
    M = max(m for m, _, _ in parts)
    L = sum(np.exp(m - M) * l for m, l, _ in parts)
    o = sum(np.exp(m - M) * oj for m, _, oj in parts)
    return o / L


# ----------------------------------------------------------------------------------------------
# AQUA with H2O token eviction [h2o], AQUA-Memory cut [mem].  One KV group at a time.
# Readings (the pages only name H2O): per KV group the attended set is the `heavy` tokens of
# largest cumulative mass (ties: lower position first) among the non-recent ones, plus the
# `recent` newest tokens (the new token included); after attending, every attended token's mass
# grows by the sum over the group's query heads of its softmax probability.  The initial mass
# comes from one full-context decode of a seeding query per head.
# ----------------------------------------------------------------------------------------------
def h2o_seed_mass(qp_heads, masks, Kp, V, scale):
    """mass[t] = sum_h p_h(t) of one full-context decode; qp_heads, masks [G][d]."""
    mass = np.zeros(Kp.shape[0])
    for h in range(qp_heads.shape[0]):
        _, p = attend(qp_heads[h], masks[h], Kp, V, scale)
        mass += p
    return mass


def h2o_heavy_set(mass, t_new, heavy, recent):
    """Positions of the heavy hitters among candidates [0, t_new - recent]: top `heavy` by
    (mass descending, position ascending)."""
    cand = np.arange(0, t_new - recent + 1)
    order = np.lexsort((cand, -mass[cand]))
    return np.sort(cand[order[:heavy]])


def h2o_step(qp_heads, masks, Kp_all, V_all, mass, t_new, heavy, recent, scale):
    """One step for the token at position t_new (rows 0..t_new of Kp_all/V_all exist; mass has
    an entry for each, the new token's being 0).  Returns (out [G][dv], new mass, attended set)."""
    H = h2o_heavy_set(mass, t_new, heavy, recent)
    A = np.concatenate([H, np.arange(max(0, t_new - recent + 1), t_new + 1)])
    out = np.zeros((qp_heads.shape[0], V_all.shape[-1]))
    add = np.zeros(A.size)
    for h in range(qp_heads.shape[0]):
        out[h], p = attend(qp_heads[h], masks[h], Kp_all[A], V_all[A], scale)
        add += p
    new_mass = mass.copy()
    new_mass[A] += add
    return out, new_mass, A


def h2o_run(P, q_seed, q_steps, K_ctx, V_ctx, k_steps, v_steps, d_sel, k, d_store, heavy,
            recent, scale, kv_dtype="f64", masks_seed=None, masks_steps=None):
    """Full-recompute run for one KV group.  q_seed [G][d]; q_steps [S][G][d];
    K_ctx, V_ctx [T][d]; k_steps, v_steps [S][d] (raw stored values).  Optional masks (e.g. from
    the GPU's q') replace the oracle's own selection.  Returns (outs [S][G][dv], attended sets,
    masses after each step)."""
    Kp = project_keys_stored(K_ctx, P, kv_dtype, d_store)
    Vc = np.asarray(V_ctx, np.float64)
    qs = project(q_seed, P)
    ms = select(qs, d_sel, k) if masks_seed is None else masks_seed
    mass = h2o_seed_mass(qs, ms, Kp, Vc, scale)
    T = Kp.shape[0]
    outs, sets, masses = [], [], []
    for s in range(q_steps.shape[0]):
        t_new = T + s
        Kp = np.concatenate([Kp, project_keys_stored(k_steps[s:s + 1], P, kv_dtype, d_store)])
        Vc = np.concatenate([Vc, np.asarray(v_steps[s:s + 1], np.float64)])
        mass = np.concatenate([mass, [0.0]])
        qp = project(q_steps[s], P)
        m = select(qp, d_sel, k) if masks_steps is None else masks_steps[s]
        o, mass, A = h2o_step(qp, m, Kp, Vc, mass, t_new, heavy, recent, scale)
        outs.append(o)
        sets.append(A)
        masses.append(mass.copy())
    return np.stack(outs), sets, masses


# ----------------------------------------------------------------------------------------------
# Offline projection [off]: P from an SVD of a calibration set.  Readings (the pages name only
# "SVD on a calibration dataset"): the set is the rows of `samples` (the stacked query and key
# vectors of one head group); P's columns are the right singular vectors in decreasing order of
# singular value, so that dim i of q' = q P is the i-th most important direction (the order the
# static memory cut relies on); the SVD leaves each column's sign free, and it is fixed here so
# that the column's entry of largest magnitude (the first such, on ties) is positive.
# ----------------------------------------------------------------------------------------------
def calibrate(samples: np.ndarray) -> np.ndarray:
    X = np.asarray(samples, dtype=np.float64)
    # rows of vt: descending singular values (all d of them; fewer samples than d need the full
    # factorisation for the directions the samples do not reach)
    _, _, vt = np.linalg.svd(X, full_matrices=X.shape[0] < X.shape[1])
    P = vt.T.copy()
    lead = np.argmax(np.abs(P), axis=0)
    P *= np.sign(P[lead, np.arange(P.shape[1])])
    return P
