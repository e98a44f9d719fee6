"""Seeded synthetic inputs shaped like one Llama-3.1-8B attention layer.

Recipe (the same for every consumer):

* P is the Q factor of a QR factorisation of a seeded d x d N(0,1) matrix, with the column signs
  chosen so that diag(R) > 0.  The fp64 matrix is kept for pins; the stored matrix is its fp32
  rounding (round to nearest even).
* Raw queries and keys are Z * diag(s) * P^T with Z ~ N(0,1) and s_i = exp(-i/tau) + 0.05,
  i = 0..d-1 (0-based).  Their projected-space value Z * diag(s) is returned as a master copy.
* Values are N(0,1).
* Stored tensors are rounded fp64 -> fp32 -> storage dtype, each step round-to-nearest-even.

Every block of rows draws from its own counter-free stream, keyed by (config id, tensor name,
batch, head[, step]), so that a sample of heads can be regenerated without the whole tensor.

This module holds no part of the attention method: it never projects for the method, selects,
scores or normalises.  The rotation by P^T above only shapes the input distribution.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# Shapes of the five workloads.  Names say what each workload is.
CONFIGS = {
    1: dict(name="tiny_decode_f32", B=1, Hq=1, Hkv=1, d=64, T=256, k=48, d_store=64, d_sel=64,
            tau=16.0, dtype="f32"),
    2: dict(name="llama8b_decode_bf16_b16_t8192", B=16, Hq=32, Hkv=8, d=128, T=8192, k=96,
            d_store=128, d_sel=128, tau=40.0, dtype="bf16"),
    3: dict(name="llama8b_long_decode_bf16_t131072", B=1, Hq=32, Hkv=8, d=128, T=131072, k=96,
            ks=(128, 96, 64, 32), d_store=128, d_sel=128, tau=40.0, dtype="bf16"),
    4: dict(name="llama8b_chunked_prefill_bf16_t16384", B=1, Hq=32, Hkv=8, d=128, T=16384,
            chunk=2048, k=96, d_store=128, d_sel=128, tau=40.0, dtype="bf16"),
    5: dict(name="llama8b_h2o_memory_bf16_t32768", B=1, Hq=32, Hkv=8, d=128, T=32768, k=64,
            d_store=96, d_sel=96, heavy=1024, recent=256, steps=64, tau=40.0, dtype="bf16"),
}

_TENSOR_IDS = {"P": 1, "q": 2, "k": 3, "v": 4, "q_step": 5, "k_step": 6, "v_step": 7, "q_seed": 8,
               "calib_q": 9, "calib_k": 10}  # calib_*: samples for the offline projection


def config(cid: int, **overrides) -> dict:
    c = dict(CONFIGS[cid])
    c["id"] = cid
    c.update(overrides)
    return c


def rng_for(cid: int, tensor: str, *idx: int) -> np.random.Generator:
    """An independent PCG64 stream for one block of one tensor."""
    ss = np.random.SeedSequence([1000 + int(cid), _TENSOR_IDS[tensor], *[int(i) for i in idx]])
    return np.random.Generator(np.random.PCG64(ss))


def decay(d: int, tau: float) -> np.ndarray:
    return np.exp(-np.arange(d, dtype=np.float64) / tau) + 0.05


def make_projection(cid: int, d: int) -> np.ndarray:
    """fp64 orthogonal P (Q of QR of a seeded Gaussian, diag(R) > 0)."""
    a = rng_for(cid, "P").standard_normal((d, d))
    q, r = np.linalg.qr(a)
    sgn = np.sign(np.diag(r))
    sgn[sgn == 0] = 1.0
    return q * sgn[None, :]


def make_qk_block(cid: int, tensor: str, idx: tuple, n: int, d: int, tau: float,
                  P64: np.ndarray):
    """(raw fp64 [n][d], projected-space master fp64 [n][d]) for one block of rows."""
    z = rng_for(cid, tensor, *idx).standard_normal((n, d))
    master = z * decay(d, tau)[None, :]
    return master @ P64.T, master


def make_v_block(cid: int, tensor: str, idx: tuple, n: int, d: int) -> np.ndarray:
    return rng_for(cid, tensor, *idx).standard_normal((n, d))


def to_storage(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """fp64 -> fp32 -> storage dtype, each step round-to-nearest-even (CPU tensor)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def storage_to_f64(t: torch.Tensor) -> np.ndarray:
    """The exact stored values, widened to fp64."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _pool_map(fn, items, workers):
    if workers <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def make_decode_inputs(c: dict, groups=None, keep_master: bool = False, workers: int = 8) -> dict:
    """Inputs of one decode step over a context of c['T'] tokens.

    Returns stored tensors q [B][Hq][d], k [B][Hkv][T][d], v [B][Hkv][T][d] (CPU, storage dtype),
    P (fp32 tensor) and P64 (fp64 numpy).  The last token T-1 is the one a decode step appends.
    With `groups` = list of (b, g), only those KV groups (and their G query heads) are drawn and
    the tensors are [len(groups)][G][d], [len(groups)][T][d], [len(groups)][T][d].
    """
    cid, B, Hq, Hkv, d, T, tau, dt = (c["id"], c["B"], c["Hq"], c["Hkv"], c["d"], c["T"],
                                      c["tau"], c["dtype"])
    G = Hq // Hkv
    P64 = make_projection(cid, d)
    out = {"P64": P64, "P": torch.from_numpy(P64.astype(np.float32)), "cfg": c}
    gl = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else list(groups)

    def one(bg):
        b, g = bg
        qs, qm = [], []
        for h in range(g * G, (g + 1) * G):
            raw, m = make_qk_block(cid, "q", (b, h), 1, d, tau, P64)
            qs.append(raw[0])
            qm.append(m[0])
        kr, km = make_qk_block(cid, "k", (b, g), T, d, tau, P64)
        vr = make_v_block(cid, "v", (b, g), T, d)
        return (to_storage(np.stack(qs), dt), to_storage(kr, dt), to_storage(vr, dt),
                (np.stack(qm), km) if keep_master else None)

    res = _pool_map(one, gl, workers)
    q = torch.stack([r[0] for r in res])
    k = torch.stack([r[1] for r in res])
    v = torch.stack([r[2] for r in res])
    if groups is None:
        q = q.reshape(B, Hkv * G, d)
        k = k.reshape(B, Hkv, T, d)
        v = v.reshape(B, Hkv, T, d)
    out.update(q=q, k=k, v=v)
    if keep_master:
        qm = np.stack([r[3][0] for r in res])
        km = np.stack([r[3][1] for r in res])
        if groups is None:
            qm = qm.reshape(B, Hkv * G, d)
            km = km.reshape(B, Hkv, T, d)
        out.update(q_master=qm, k_master=km)
    return out


def make_prefill_inputs(c: dict, heads=None, rows=None, workers: int = 8) -> dict:
    """Inputs of a causal prefill over T tokens: q [B][Hq][T][d], k, v [B][Hkv][T][d].

    `heads` restricts q to a list of (b, h); `rows` then restricts each head to those positions
    (the full block is still drawn so that values agree with the full tensor).
    """
    cid, B, Hq, Hkv, d, T, tau, dt = (c["id"], c["B"], c["Hq"], c["Hkv"], c["d"], c["T"],
                                      c["tau"], c["dtype"])
    P64 = make_projection(cid, d)
    out = {"P64": P64, "P": torch.from_numpy(P64.astype(np.float32)), "cfg": c}
    hl = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)

    def qblock(bh):
        raw, _ = make_qk_block(cid, "q", bh, T, d, tau, P64)
        if rows is not None:
            raw = raw[np.asarray(rows)]
        return to_storage(raw, dt)

    def kvblock(bg):
        kr, _ = make_qk_block(cid, "k", bg, T, d, tau, P64)
        return to_storage(kr, dt), to_storage(make_v_block(cid, "v", bg, T, d), dt)

    qs = _pool_map(qblock, hl, workers)
    q = torch.stack(qs)
    gl = [(b, g) for b in range(B) for g in range(Hkv)]
    kv = _pool_map(kvblock, gl, workers)
    k = torch.stack([x[0] for x in kv]).reshape(B, Hkv, T, d)
    v = torch.stack([x[1] for x in kv]).reshape(B, Hkv, T, d)
    if heads is None:
        q = q.reshape(B, Hq, q.shape[-2], d)
    out.update(q=q, k=k, v=v)
    return out


def make_h2o_inputs(c: dict, workers: int = 8) -> dict:
    """Context k, v [B][Hkv][T][d]; seeding query q_seed [B][Hq][d]; per-step tokens
    q_steps [S][B][Hq][d], k_steps / v_steps [S][B][Hkv][d] for steps 1..S."""
    cid, B, Hq, Hkv, d, T, tau, dt, S = (c["id"], c["B"], c["Hq"], c["Hkv"], c["d"], c["T"],
                                         c["tau"], c["dtype"], c["steps"])
    P64 = make_projection(cid, d)
    out = {"P64": P64, "P": torch.from_numpy(P64.astype(np.float32)), "cfg": c}
    gl = [(b, g) for b in range(B) for g in range(Hkv)]

    def kvblock(bg):
        kr, _ = make_qk_block(cid, "k", bg, T, d, tau, P64)
        return to_storage(kr, dt), to_storage(make_v_block(cid, "v", bg, T, d), dt)

    kv = _pool_map(kvblock, gl, workers)
    out["k"] = torch.stack([x[0] for x in kv]).reshape(B, Hkv, T, d)
    out["v"] = torch.stack([x[1] for x in kv]).reshape(B, Hkv, T, d)
    qs = [make_qk_block(cid, "q_seed", (b, h), 1, d, tau, P64)[0][0]
          for b in range(B) for h in range(Hq)]
    out["q_seed"] = to_storage(np.stack(qs).reshape(B, Hq, d), dt)
    qst, kst, vst = [], [], []
    for s in range(1, S + 1):
        qst.append(np.stack([make_qk_block(cid, "q_step", (s, b, h), 1, d, tau, P64)[0][0]
                             for b in range(B) for h in range(Hq)]).reshape(B, Hq, d))
        kst.append(np.stack([make_qk_block(cid, "k_step", (s, b, g), 1, d, tau, P64)[0][0]
                             for b in range(B) for g in range(Hkv)]).reshape(B, Hkv, d))
        vst.append(np.stack([make_v_block(cid, "v_step", (s, b, g), 1, d)[0]
                             for b in range(B) for g in range(Hkv)]).reshape(B, Hkv, d))
    out["q_steps"] = to_storage(np.stack(qst), dt)
    out["k_steps"] = to_storage(np.stack(kst), dt)
    out["v_steps"] = to_storage(np.stack(vst), dt)
    return out
