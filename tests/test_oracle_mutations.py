"""Planted mistakes in the oracle (CPU only): each must make at least one pin fail.

This checks that the pins have teeth: a dropped term, a wrong sign, index or orientation anywhere
in the oracle is caught by something other than the oracle itself.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import aqua_oracle as O

_orig = {name: getattr(O, name) for name in O.__all__}


def _select_ties_high(qp, d_sel, k):
    qp = np.asarray(qp, np.float64)
    d = qp.shape[-1]
    rows = qp.reshape(-1, d)
    mask = np.zeros(rows.shape, bool)
    for r in range(rows.shape[0]):
        mag = np.abs(rows[r, :d_sel])
        order = np.lexsort((-np.arange(d_sel), -mag))  # ties: higher index first
        mask[r, order[:k]] = True
    return mask.reshape(qp.shape)


def _select_smallest(qp, d_sel, k):
    return _orig["select"](1.0 / (np.abs(qp) + 1e-300), d_sel, k)


def _select_signed(qp, d_sel, k):
    # ranks by signed value instead of magnitude
    qp = np.asarray(qp, np.float64)
    return _orig["select"](np.where(qp > 0, qp, 0.0) + 1e-300 * np.arange(qp.shape[-1])[::-1],
                           d_sel, k)


def _project_transposed(x, P):
    return np.asarray(x, np.float64) @ np.asarray(P, np.float64).T


def _scores_all_dims(qp_row, mask_row, Kp, scale):
    return (Kp @ qp_row[:Kp.shape[-1]]) * float(scale)


def _scores_no_scale(qp_row, mask_row, Kp, scale):
    return _orig["sparse_scores"](qp_row, mask_row, Kp, 1.0)


def _scores_sqrt_k_scale(qp_row, mask_row, Kp, scale):
    k = int(np.sum(mask_row))
    return _orig["sparse_scores"](qp_row, mask_row, Kp, 1.0 / np.sqrt(k))


def _decode_gqa_mod(qp, mask, Kp, V, scale, length=None, return_p=False):
    B, Hq, _ = qp.shape
    Hkv = Kp.shape[1]
    T = Kp.shape[2] if length is None else int(length)
    out = np.zeros((B, Hq, V.shape[-1]))
    ps = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h % Hkv
            out[b, h], ps[b, h] = O.attend(qp[b, h], mask[b, h], Kp[b, g, :T], V[b, g, :T], scale)
    return (out, ps) if return_p else out


def _prefill_exclusive(qp, mask, Kp, V, positions, scale):
    return _orig["prefill"](qp, mask, Kp, V, np.maximum(np.asarray(positions) - 1, 0), scale)


def _combine_unweighted(parts):
    return sum(o for _, _, o in parts) / sum(l for _, l, _ in parts)


def _heavy_ties_late(mass, t_new, heavy, recent):
    cand = np.arange(0, t_new - recent + 1)
    order = np.lexsort((-cand, -mass[cand]))
    return np.sort(cand[order[:heavy]])


def _h2o_step_one_head(qp_heads, masks, Kp_all, V_all, mass, t_new, heavy, recent, scale):
    out, new_mass, A = _orig["h2o_step"](qp_heads, masks, Kp_all, V_all, mass, t_new, heavy,
                                         recent, scale)
    _, p0 = O.attend(qp_heads[0], masks[0], Kp_all[A], V_all[A], scale)
    m = mass.copy()
    m[A] += p0
    return out, m, A


def _round_truncate(x, dtype):
    if dtype != "bf16":
        return _orig["round_to_storage"](x, dtype)
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.trunc(x / q) * q


def _softmax_unnormalised(s):
    return np.exp(s - np.max(s))


def _memory_cut_last_dims(K, P, dtype, d_store):
    return _orig["round_to_storage"](_orig["project"](K, P), dtype)[..., -d_store:]


def _calibrate_ascending(samples):
    return _orig["calibrate"](samples)[:, ::-1]


def _calibrate_left_vectors(samples):
    # the left singular vectors' first d rows instead of the right singular vectors
    X = np.asarray(samples, np.float64)
    u, _, _ = np.linalg.svd(X, full_matrices=False)
    d = X.shape[1]
    return u[:d, :d] if u.shape[0] >= d else np.eye(d)


def _calibrate_transposed(samples):
    return _orig["calibrate"](samples).T


MUTANTS = {
    "calibrate: ascending singular values": ("calibrate", _calibrate_ascending),
    "calibrate: left singular vectors": ("calibrate", _calibrate_left_vectors),
    "calibrate: P transposed": ("calibrate", _calibrate_transposed),
    "select: ties to the higher index": ("select", _select_ties_high),
    "select: smallest magnitudes": ("select", _select_smallest),
    "select: signed value, not magnitude": ("select", _select_signed),
    "project: x P^T instead of x P": ("project", _project_transposed),
    "scores: every dim, mask ignored": ("sparse_scores", _scores_all_dims),
    "scores: scale dropped": ("sparse_scores", _scores_no_scale),
    "scores: 1/sqrt(k) scale": ("sparse_scores", _scores_sqrt_k_scale),
    "decode: head h reads KV head h mod Hkv": ("decode", _decode_gqa_mod),
    "prefill: causal bound exclusive": ("prefill", _prefill_exclusive),
    "combine: partials not rescaled": ("combine_partials", _combine_unweighted),
    "h2o: ties to the later position": ("h2o_heavy_set", _heavy_ties_late),
    "h2o: mass from one head only": ("h2o_step", _h2o_step_one_head),
    "storage: bf16 truncation": ("round_to_storage", _round_truncate),
    "softmax: not normalised": ("softmax", _softmax_unnormalised),
    "memory cut: last dims kept": ("project_keys_stored", _memory_cut_last_dims),
}


@pytest.mark.filterwarnings("ignore::UserWarning")
@pytest.mark.parametrize("label", sorted(MUTANTS))
def test_planted_mistake_is_caught(label, monkeypatch):
    name, fn = MUTANTS[label]
    monkeypatch.setattr(O, name, fn)
    failed = []
    for pin_name, pin in oracle_pins.PINS.items():
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin_name)
    assert failed, f"no pin catches: {label}"
