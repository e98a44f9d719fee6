"""Helpers for the GPU parity tests: run libaqua through its C ABI, compare with the oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

import sparse_dimension_attention_amd as aq
from oracle import aqua_oracle as O
from synth import storage_to_f64

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

F32_TOL = 1e-5                  # max-abs, fp32 storage
BF16_MAXABS, BF16_RELL2 = 1e-2, 5e-3
U = 2.0 ** -24                  # fp32 unit roundoff


def gamma(n):
    return n * U / (1 - n * U)


def mass_tol(qp, m, Kp, scale, k):
    """Relative bound on the GPU's softmax weights against fp64 weights computed from the GPU's
    own q' and K' (no figure is given for it, so it is derived from the fp32 arithmetic).
    qp, m [G][d] (GPU q', masks); Kp [n][d_store] (GPU K', token-major).  A score error
    |ds| <= gamma_(k+2) * scale * sum_i |q'_i K'_i| moves a weight by a factor
    exp(ds_t - sum_u p_u ds_u), i.e. relative error <= 2 max|ds|; the log2-domain subtraction
    s - max s (|s - m| <= 2 S log2 e) rounds once more, and exp2, the division and the fp32
    additions a few u."""
    S = scale * float((np.abs(qp[:, :Kp.shape[1]] * m[:, :Kp.shape[1]]) @ np.abs(Kp).T).max())
    return 2 * gamma(k + 2) * S + 6 * U * S + 8 * U


def check_mass_update(before, after, add, tol, what=""):
    """after = before + add per element, in fp32: |after - (before + add)| must stay within the
    weights' relative bound tol * add plus the rounding of the fp32 sum, 2u (before + add)."""
    before, after, add = (np.asarray(x, np.float64) for x in (before, after, add))
    want = before + add
    dm = np.abs(after - want)
    lim = tol * add + 2 * U * np.abs(want)
    assert np.all(dm <= lim), f"{what}: mass error / bound {float(np.max(dm / lim))}"


def unpack_mask(mask_i32: torch.Tensor, d: int) -> np.ndarray:
    """[..., d/32] int32 words -> bool [..., d] (bit i % 32 of word i / 32)."""
    a = mask_i32.detach().cpu().contiguous().numpy()
    bits = np.unpackbits(a.view(np.uint8), bitorder="little")
    return bits.reshape(*a.shape[:-1], d).astype(bool)


def rel_l2(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def assert_close(x, ref, dtype, what=""):
    err = float(np.max(np.abs(x - ref)))
    if dtype == "f32":
        assert err < F32_TOL, f"{what} max-abs {err}"
    else:
        r = rel_l2(x, ref)
        assert err < BF16_MAXABS and r < BF16_RELL2, f"{what} max-abs {err}, rel-L2 {r}"
    return err


def tdtype(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def new_cache(B, Hkv, d, d_store, T_cap, dtype):
    """NaN-poisoned K' [B][Hkv][d_store][T_cap] and V [B][Hkv][T_cap][d] on the GPU."""
    kp = torch.full((B, Hkv, d_store, T_cap), float("nan"), dtype=tdtype(dtype), device=DEV)
    v = torch.full((B, Hkv, T_cap, d), float("nan"), dtype=tdtype(dtype), device=DEV)
    return kp, v


def kp_token_major(kp, b, g, length):
    """The GPU's K' of group (b, g), tokens [0, length), as fp64 [length][d_store]."""
    return kp[b, g, :, :length].T.cpu().double().numpy()


def select(q_dev, P_dev, d_sel, k, want_idx=False):
    N, d = q_dev.shape
    qp = torch.full((N, d), float("nan"), device=DEV)
    mask = torch.full((N, d // 32), -1, dtype=torch.int32, device=DEV)
    idx = torch.full((N, k), -1, dtype=torch.int16, device=DEV) if want_idx else None
    aq.aqua_select_dims(q_dev, P_dev, d_sel, k, qp, mask, idx)
    return qp, mask, idx


def run_decode(inp, c, length=None, T_cap=None, k=None, d_store=None, d_sel=None, mass=None):
    """The decode path on the GPU: append K'/V for the context, select, decode.
    Returns GPU tensors (out, q', mask) and the cache tensors."""
    B, Hq, Hkv, d = c["B"], c["Hq"], c["Hkv"], c["d"]
    T = inp["k"].shape[2] if length is None else length
    T_cap = T_cap or ((T + 63) // 64 * 64)
    k = c["k"] if k is None else k
    d_store = c.get("d_store", d) if d_store is None else d_store
    d_sel = c.get("d_sel", d) if d_sel is None else d_sel
    kp, v = new_cache(B, Hkv, d, d_store, T_cap, c["dtype"])
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T].contiguous().to(DEV),
                         inp["v"][:, :, :T].contiguous().to(DEV), P, T)
    assert cache.len == T
    qp, mask, _ = select(inp["q"].reshape(B * Hq, d).to(DEV), P, d_sel, k)
    ws = torch.zeros(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp, mask, 1 / math.sqrt(d), out, ws, mass=mass)
    torch.cuda.synchronize()
    return dict(out=out, qp=qp.reshape(B, Hq, d), mask=mask.reshape(B, Hq, d // 32), kp=kp, v=v,
                cache=cache, ws=ws, P=P)


def oracle_decode(inp, c, mask_np, length=None, d_store=None, heads=None):
    """Oracle output for the stored inputs with the given (GPU-derived) masks.
    heads: optional list of (b, h) to compute (others left NaN)."""
    B, Hq, Hkv, d = c["B"], c["Hq"], c["Hkv"], c["d"]
    G = Hq // Hkv
    T = inp["k"].shape[2] if length is None else length
    d_store = c.get("d_store", d) if d_store is None else d_store
    P64 = storage_to_f64(inp["P"])
    qp64 = O.project(storage_to_f64(inp["q"]), P64)
    out = np.full((B, Hq, d), np.nan)
    hl = heads or [(b, h) for b in range(B) for h in range(Hq)]
    groups = sorted({(b, h // G) for b, h in hl})
    for b, g in groups:
        Kp = O.project_keys_stored(storage_to_f64(inp["k"][b, g, :T]), P64, c["dtype"], d_store)
        V = storage_to_f64(inp["v"][b, g, :T])
        for bb, h in hl:
            if bb == b and h // G == g:
                out[b, h], _ = O.attend(qp64[b, h], mask_np[b, h], Kp, V, 1 / math.sqrt(d))
    return out
