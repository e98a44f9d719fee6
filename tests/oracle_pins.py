"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin is a plain function that raises AssertionError when the oracle disagrees with:
  * values worked by hand (tests/golden/*.json),
  * closed forms of the synthetic generator,
  * library routines computing a special case (torch's fp64 scaled_dot_product_attention),
  * brute force on tiny inputs written as loops, with a different selection algorithm,
  * invariants of the definition.

The pins look the oracle's functions up on the module at call time, so a test can swap one of
them for a plausible mistake and check that some pin fails.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

from oracle import aqua_oracle as O
from synth import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, v, scale, gqa=False, attn_mask=None):
    """torch fp64 attention: q [B][H][L][d], k/v [B][Hkv][T][d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # noqa: E731
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if attn_mask is None else torch.from_numpy(attn_mask),
        scale=scale, enable_gqa=gqa)
    return o.numpy()


def _decode_via_oracle(q_raw, K_raw, V, P, d_sel, k, scale, kv_dtype="f64", d_store=None):
    """The whole decode path through the oracle: project, select, store K', attend."""
    d = q_raw.shape[-1]
    ds = d if d_store is None else d_store
    qp = O.project(q_raw, P)
    m = O.select(qp, d_sel, k)
    Kp = O.project_keys_stored(K_raw, P, kv_dtype, ds)
    return O.decode(qp, m, Kp, V, scale), qp, m, Kp


# ---------------------------------------------------------------- storage rounding
def pin_bf16_rounding():
    rng = _rng(1)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    # exact halfway cases between neighbouring bf16 values: ties must go to the even one
    base = torch.tensor(rng.standard_normal(2000), dtype=torch.float32).to(torch.bfloat16)
    b = base.to(torch.float32).numpy().astype(np.float64)
    _, e = np.frexp(b)
    half = np.ldexp(1.0, e - 9)
    halves = (b + half).astype(np.float32)
    sub = (np.arange(-300, 300) * 2.0 ** -140).astype(np.float32)  # bf16 subnormal range
    for xs in (x32, halves, sub):
        want = torch.from_numpy(xs).to(torch.bfloat16).to(torch.float64).numpy()
        got = O.round_to_storage(xs.astype(np.float64), "bf16")
        assert np.array_equal(got, want), "bf16 rounding disagrees with torch's fp32->bf16"
    x = rng.standard_normal(1000)
    assert np.array_equal(O.round_to_storage(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- projection
def pin_projection_orthogonal():
    P64 = gen.make_projection(2, 128)
    rng = _rng(2)
    q = rng.standard_normal((50, 128))
    qp = O.project(q, P64)
    assert np.allclose(np.linalg.norm(qp, axis=1), np.linalg.norm(q, axis=1), rtol=1e-12, atol=0)
    assert np.allclose(qp @ P64.T, q, rtol=0, atol=1e-12)


def pin_generator_closed_form():
    """Raw = Z diag(s) P^T, so the oracle's q' = raw P must give back Z diag(s)."""
    for cid in (1, 2):
        c = gen.config(cid)
        P64 = gen.make_projection(cid, c["d"])
        raw, master = gen.make_qk_block(cid, "k", (0, 0), 64, c["d"], c["tau"], P64)
        assert np.allclose(O.project(raw, P64), master, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- selection
def _check_characterisation(q, mask, d_sel, k):
    a = np.abs(q)
    S = [i for i in range(d_sel) if mask[i]]
    N = [j for j in range(d_sel) if not mask[j]]
    assert len(S) == k and not mask[d_sel:].any()
    for i in S:
        for j in N:
            assert a[i] > a[j] or (a[i] == a[j] and i < j)


def pin_select_golden():
    with open(os.path.join(GOLDEN, "select_ties.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = O.select(np.array([c["q"]]), c["d_sel"], c["k"])[0]
        assert list(got) == c["mask"], c["why"]


def pin_select_characterisation():
    rng = _rng(3)
    for d, d_sel, k in [(64, 64, 48), (128, 128, 96), (128, 96, 64), (128, 128, 1), (128, 128, 128)]:
        q = rng.standard_normal((20, d)) * np.exp(-np.arange(d) / 40)
        q[0, :] = np.round(q[0, :] * 4) / 4  # many exact ties
        m = O.select(q, d_sel, k)
        for r in range(q.shape[0]):
            _check_characterisation(q[r], m[r], d_sel, k)


def pin_select_bruteforce():
    """Over every k-subset of the eligible dims exactly one satisfies the selection rule, and it
    is the oracle's.  Values from a small set so that ties are frequent."""
    rng = _rng(4)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 0.5])
    for _ in range(60):
        d = int(rng.integers(2, 9))
        d_sel = int(rng.integers(1, d + 1))
        k = int(rng.integers(1, d_sel + 1))
        q = rng.choice(vals, size=d)
        a = np.abs(q)
        good = []
        for S in itertools.combinations(range(d_sel), k):
            rest = [j for j in range(d_sel) if j not in S]
            if all(a[i] > a[j] or (a[i] == a[j] and i < j) for i in S for j in rest):
                good.append(S)
        assert len(good) == 1
        want = np.zeros(d, bool)
        want[list(good[0])] = True
        assert np.array_equal(O.select(q[None], d_sel, k)[0], want)


# ---------------------------------------------------------------- attention special cases
def pin_hand_example():
    with open(os.path.join(GOLDEN, "hand_d4.json")) as f:
        g = json.load(f)
    P = np.eye(g["d"])
    out, qp, m, Kp = _decode_via_oracle(np.array([[g["q"]]]), np.array([[g["K"]]]),
                                        np.array([[g["V"]]]), P, g["d"], g["k"],
                                        1 / math.sqrt(g["d"]))
    assert list(m[0, 0]) == g["mask"]
    _, p = O.attend(qp[0, 0], m[0, 0], Kp[0, 0], np.array(g["V"]), 1 / math.sqrt(g["d"]))
    assert np.allclose(p, g["p"], rtol=0, atol=1e-14)
    assert np.allclose(out[0, 0], g["out"], rtol=0, atol=1e-13)


def pin_k_equals_d_is_exact_attention():
    """With k = d and orthogonal fp64 P, AQUA is exactly softmax(q K^T / sqrt d) V on the raw
    vectors (the rotation cancels).  Checked against torch's fp64 SDPA, GQA included."""
    for cid, B, Hq, Hkv, d, T in [(1, 1, 1, 1, 64, 256), (2, 2, 8, 2, 128, 300)]:
        c = gen.config(cid)
        P64 = gen.make_projection(cid, d)
        rng = _rng(5)
        q = np.stack([np.stack([gen.make_qk_block(cid, "q", (b, h), 1, d, c["tau"], P64)[0][0]
                                for h in range(Hq)]) for b in range(B)])
        K = np.stack([np.stack([gen.make_qk_block(cid, "k", (b, g), T, d, c["tau"], P64)[0]
                                for g in range(Hkv)]) for b in range(B)])
        V = rng.standard_normal((B, Hkv, T, d))
        out, *_ = _decode_via_oracle(q, K, V, P64, d, d, 1 / math.sqrt(d))
        ref = _sdpa(q[:, :, None, :], K, V, 1 / math.sqrt(d), gqa=(Hq != Hkv))[:, :, 0, :]
        assert np.max(np.abs(out - ref)) < 1e-10


def pin_masked_query_identity():
    """For any k: the sparse score equals the full dot product of the zero-masked q' with K', so
    AQUA = SDPA(q' * mask, K', V) with scale 1/sqrt(d).  Pins scores, scale, softmax, GQA map."""
    rng = _rng(6)
    B, Hq, Hkv, d, T = 2, 8, 2, 32, 40
    P = gen.make_projection(7, d)
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    for k in (1, 5, 24, 32):
        out, qp, m, Kp = _decode_via_oracle(q, K, V, P, d, k, 1 / math.sqrt(d))
        ref = _sdpa((qp * m)[:, :, None, :], Kp, V, 1 / math.sqrt(d), gqa=True)[:, :, 0, :]
        assert np.max(np.abs(out - ref)) < 1e-12


def pin_identity_projection():
    """P = I: scores use the k raw dims of largest |q| (selected here by a full sort written
    independently)."""
    rng = _rng(8)
    d, T, k = 8, 12, 3
    q = rng.standard_normal((1, 1, d))
    K = rng.standard_normal((1, 1, T, d))
    V = rng.standard_normal((1, 1, T, d))
    out, *_ = _decode_via_oracle(q, K, V, np.eye(d), d, k, 0.25)
    top = sorted(range(d), key=lambda i: (-abs(q[0, 0, i]), i))[:k]
    qm = np.zeros(d)
    qm[top] = q[0, 0, top]
    ref = _sdpa(qm[None, None, None, :], K, V, 0.25)[0, 0, 0]
    assert np.max(np.abs(out[0, 0] - ref)) < 1e-13


def pin_softmax_invariants():
    rng = _rng(9)
    d, T = 16, 50
    P = gen.make_projection(9, d)
    q = rng.standard_normal((1, 2, d))
    K = rng.standard_normal((1, 1, T, d)) * 3
    V = rng.standard_normal((1, 1, T, d))
    qp = O.project(q, P)
    m = O.select(qp, d, 7)
    Kp = O.project_keys_stored(K, P, "f64", d)
    out, ps = O.decode(qp, m, Kp, V, 0.25, return_p=True)
    assert np.allclose(ps.sum(-1), 1.0, rtol=0, atol=1e-14) and (ps >= 0).all()
    out2 = O.decode(qp, m, Kp, V + 3.5, 0.25)
    assert np.allclose(out2, out + 3.5, rtol=0, atol=1e-13)
    perm = rng.permutation(T)
    out3 = O.decode(qp, m, Kp[:, :, perm], V[:, :, perm], 0.25)
    assert np.allclose(out3, out, rtol=0, atol=1e-13)


def _bruteforce_decode(q_raw, K_raw, V, P, k, scale):
    """Scalar loops: projection by explicit sums, selection by counting how many dims beat each
    dim, scores over the selected dims, softmax with math.exp, weighted sum."""
    B, Hq, d = q_raw.shape
    Hkv, T = K_raw.shape[1], K_raw.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, V.shape[-1]))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qp = [sum(q_raw[b, h, j] * P[j, i] for j in range(d)) for i in range(d)]
            keep = []
            for i in range(d):
                beaten_by = sum(1 for j in range(d)
                                if abs(qp[j]) > abs(qp[i]) or (abs(qp[j]) == abs(qp[i]) and j < i))
                keep.append(beaten_by < k)
            s = []
            for t in range(T):
                kp = [sum(K_raw[b, g, t, j] * P[j, i] for j in range(d)) for i in range(d)]
                s.append(scale * sum(qp[i] * kp[i] for i in range(d) if keep[i]))
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for c in range(V.shape[-1]):
                out[b, h, c] = sum(e[t] / z * V[b, g, t, c] for t in range(T))
    return out


def pin_bruteforce_tiny():
    rng = _rng(10)
    for d, T, Hq, Hkv, k in [(4, 5, 1, 1, 2), (8, 16, 4, 2, 3), (8, 9, 4, 1, 8), (4, 16, 2, 2, 1)]:
        P = gen.make_projection(11, d)
        q = rng.standard_normal((2, Hq, d))
        K = rng.standard_normal((2, Hkv, T, d))
        V = rng.standard_normal((2, Hkv, T, d))
        out, *_ = _decode_via_oracle(q, K, V, P, d, k, 1 / math.sqrt(d))
        ref = _bruteforce_decode(q, K, V, P, k, 1 / math.sqrt(d))
        assert np.max(np.abs(out - ref)) < 1e-13


# ---------------------------------------------------------------- prefill / chunking / splits
def pin_prefill_equals_decode():
    """The prefill row at position p equals a decode over the first p+1 tokens."""
    rng = _rng(12)
    B, Hq, Hkv, d, T = 1, 4, 2, 16, 24
    P = gen.make_projection(12, d)
    q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    qp = O.project(q, P)
    m = O.select(qp, d, 10)
    Kp = O.project_keys_stored(K, P, "f64", d)
    full = O.prefill(qp, m, Kp, V, np.arange(T), 0.25)
    for p in (0, 1, 7, T - 1):
        dec = O.decode(qp[:, :, p], m[:, :, p], Kp[:, :, :p + 1], V[:, :, :p + 1], 0.25)
        assert np.allclose(full[:, :, p], dec, rtol=0, atol=1e-13)


def pin_causal_against_library():
    """Prefill with k = d equals causal SDPA on the raw vectors (fp64 P), GQA included."""
    rng = _rng(13)
    B, Hq, Hkv, d, T = 1, 4, 2, 16, 20
    P = gen.make_projection(13, d)
    q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    out = O.chunked_prefill(q, K, V, P, d, d, 1 / math.sqrt(d), chunk=T)
    causal = np.tril(np.ones((T, T), dtype=bool))
    ref = _sdpa(q, K, V, 1 / math.sqrt(d), gqa=True, attn_mask=causal)
    assert np.max(np.abs(out - ref)) < 1e-10


def pin_chunking_invariance():
    rng = _rng(14)
    B, Hq, Hkv, d, T = 1, 4, 2, 16, 23
    P = gen.make_projection(14, d)
    q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    ref = O.chunked_prefill(q, K, V, P, d, 9, 0.25, chunk=T)
    for ch in (1, 7, 16):
        out = O.chunked_prefill(q, K, V, P, d, 9, 0.25, chunk=ch)
        assert np.allclose(out, ref, rtol=0, atol=1e-12)


def pin_split_combine():
    rng = _rng(15)
    T, dv = 1000, 8
    s = rng.standard_normal(T) * 5
    s[300:400] -= 80  # a split whose scores are far below the rest
    V = rng.standard_normal((T, dv))
    p = np.exp(s - s.max())
    direct = (p / p.sum()) @ V
    for bounds in ([(0, T)], [(0, 1), (1, T)], [(0, 300), (300, 400), (400, 1000)],
                   [(i, min(T, i + 64)) for i in range(0, T, 64)]):
        got = O.combine_partials(O.split_partials(s, V, bounds))
        assert np.allclose(got, direct, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- AQUA-Memory and H2O
def pin_memory_cut():
    rng = _rng(16)
    B, Hq, Hkv, d, T = 1, 4, 1, 32, 30
    P = gen.make_projection(16, d)
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    full, *_ = _decode_via_oracle(q, K, V, P, d, 10, 0.2)
    same, *_ = _decode_via_oracle(q, K, V, P, d, 10, 0.2, d_store=d)
    assert np.array_equal(full, same)
    # k = d_sel = 24: a static cut to the first 24 projected dims
    out, qp, _, Kp = _decode_via_oracle(q, K, V, P, 24, 24, 0.2, d_store=24)
    ref = _sdpa(qp[:, :, None, :24], Kp, V, 0.2, gqa=True)[:, :, 0, :]
    assert np.max(np.abs(out - ref)) < 1e-12


def _h2o_small_inputs(seed, T, S, G, d):
    rng = _rng(seed)
    return (gen.make_projection(seed, d), rng.standard_normal((G, d)),
            rng.standard_normal((S, G, d)), rng.standard_normal((T, d)) * 2,
            rng.standard_normal((T, d)), rng.standard_normal((S, d)) * 2,
            rng.standard_normal((S, d)))


def pin_h2o_everything_kept():
    """heavy + recent covering every token: each step is a plain full-context decode."""
    T, S, G, d = 20, 6, 4, 16
    P, qs, qst, K, V, ks, vs = _h2o_small_inputs(17, T, S, G, d)
    outs, sets, _ = O.h2o_run(P, qs, qst, K, V, ks, vs, d_sel=12, k=5, d_store=12, heavy=T,
                              recent=S + 1, scale=0.25)
    for s in range(S):
        n = T + s + 1
        assert np.array_equal(sets[s], np.arange(n))
        Kp = O.project_keys_stored(np.concatenate([K, ks[:s + 1]]), P, "f64", 12)
        Vc = np.concatenate([V, vs[:s + 1]])
        qp = O.project(qst[s], P)
        m = O.select(qp, 12, 5)
        ref = _sdpa((qp * m)[None, :, None, :12], Kp[None, None], Vc[None, None], 0.25,
                    gqa=True)[0, :, 0]
        assert np.max(np.abs(outs[s] - ref)) < 1e-12


def pin_h2o_heavy_set_rule():
    """The heavy set satisfies its defining order, with ties (equal mass) broken by position."""
    rng = _rng(18)
    for _ in range(30):
        n = int(rng.integers(5, 40))
        mass = rng.choice([0.0, 0.25, 0.5, 1.0, 2.0], size=n)
        recent = int(rng.integers(1, 4))
        heavy = int(rng.integers(1, n - recent + 1))
        t_new = n - 1
        H = set(O.h2o_heavy_set(mass, t_new, heavy, recent).tolist())
        C = range(0, t_new - recent + 1)
        assert len(H) == min(heavy, len(C))
        for x in H:
            for y in C:
                if y not in H:
                    assert mass[x] > mass[y] or (mass[x] == mass[y] and x < y)


def pin_h2o_one_eviction_form():
    """The full re-sort each step equals a fixed set of heavy + recent slots with exactly one
    eviction per step (the lowest-ranked non-recent slot), which is what a compact cache does."""
    T, S, G, d, heavy, recent = 60, 25, 2, 16, 12, 6
    P, qs, qst, K, V, ks, vs = _h2o_small_inputs(19, T, S, G, d)
    outs, sets, masses = O.h2o_run(P, qs, qst, K, V, ks, vs, d_sel=12, k=6, d_store=12,
                                   heavy=heavy, recent=recent, scale=0.25)
    # initial slots: heavy hitters of [0, T - recent] by the seeding mass, plus [T-recent+1, T-1]
    Kp = O.project_keys_stored(K, P, "f64", 12)
    qsp = O.project(qs, P)
    mass = O.h2o_seed_mass(qsp, O.select(qsp, 12, 6), Kp, V, 0.25)
    cand = np.arange(0, T - recent)
    order = np.lexsort((cand, -mass[cand]))
    slots = set(cand[order[:heavy]].tolist()) | set(range(T - recent, T))
    for s in range(S):
        t_new = T + s
        non_recent = [x for x in slots if x <= t_new - recent]
        m_prev = masses[s - 1] if s else mass
        victim = min(non_recent, key=lambda x: (m_prev[x], -x))  # least mass, then latest
        slots = (slots - {victim}) | {t_new}
        assert slots == set(sets[s].tolist()), f"step {s}"


def _bruteforce_probs(q_row, K_rows, P, d_sel, k, scale):
    """Softmax weights of one raw query over raw key rows, by scalar loops (selection by
    counting, as in the brute-force decode)."""
    d = len(q_row)
    qp = [sum(q_row[j] * P[j, i] for j in range(d)) for i in range(d)]
    keep = [i < d_sel and sum(1 for j in range(d_sel) if abs(qp[j]) > abs(qp[i])
                              or (abs(qp[j]) == abs(qp[i]) and j < i)) < k for i in range(d)]
    s = []
    for row in K_rows:
        kp = [sum(row[j] * P[j, i] for j in range(d)) for i in range(d)]
        s.append(scale * sum(qp[i] * kp[i] for i in range(d) if keep[i]))
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    z = sum(e)
    return [x / z for x in e]


def pin_h2o_mass_accounting():
    """Every step adds exactly G units of mass (one softmax per query head), only to the
    attended tokens, each token's share being the brute-force sum of the heads' weights."""
    T, S, G, d, heavy, recent, d_sel, k = 14, 5, 3, 8, 4, 3, 6, 4
    P, qs, qst, K, V, ks, vs = _h2o_small_inputs(20, T, S, G, d)
    outs, sets, masses = O.h2o_run(P, qs, qst, K, V, ks, vs, d_sel=d_sel, k=k, d_store=d_sel,
                                   heavy=heavy, recent=recent, scale=0.3)
    seed = np.zeros(T)
    for h in range(G):
        seed += np.array(_bruteforce_probs(qs[h], K, P, d_sel, k, 0.3))
    prev = seed
    for s in range(S):
        Kall = np.concatenate([K, ks[:s + 1]])
        inc = masses[s] - np.concatenate([prev, [0.0]])
        A = sets[s]
        want = np.zeros(T + s + 1)
        for h in range(G):
            want[A] += np.array(_bruteforce_probs(qst[s, h], Kall[A], P, d_sel, k, 0.3))
        assert abs(inc.sum() - G) < 1e-12
        assert np.allclose(inc, want, rtol=0, atol=1e-13), f"step {s}"
        prev = masses[s]


def pin_25_percent():
    """The pages' figure: keeping 96 of 128 dims cuts query-key products by 25 %."""
    c = gen.config(2)
    assert 1 - c["k"] / c["d"] == 0.25


def _orthonormal(rng, n, m):
    q, r = np.linalg.qr(rng.standard_normal((n, m)))
    return q * np.sign(np.diag(r))


def pin_calibrate_recovers_rotation():
    """Samples X = A diag(s) R^T with orthonormal A and distinct s have X^T X = R diag(s^2) R^T
    exactly, so the calibrated P is R column for column up to sign, in decreasing order of s."""
    rng = _rng(71)
    d, n = 16, 200
    R = _orthonormal(rng, d, d)
    s = np.sort(rng.uniform(0.5, 3.0, d))[::-1]
    perm = rng.permutation(d)  # the rows of X come in any order of the directions
    X = _orthonormal(rng, n, d)[:, perm] @ np.diag(s[perm]) @ R[:, perm].T
    P = O.calibrate(X)
    assert P.shape == (d, d)
    assert np.allclose(np.abs(P.T @ R), np.eye(d), atol=1e-10)
    # the variance of each calibrated coordinate is the matching s^2, in decreasing order
    assert np.allclose(np.sum((X @ P) ** 2, axis=0), s ** 2, rtol=1e-10)
    # the sign rule: each column's largest-magnitude entry is positive
    lead = np.argmax(np.abs(P), axis=0)
    assert np.all(P[lead, np.arange(d)] > 0)


def pin_calibrate_low_rank():
    """A rank-r calibration set: P is orthogonal, its first r columns span the samples' row space
    (X P has zero columns past r), and the calibrated coordinates carry all the energy."""
    rng = _rng(72)
    d, n, r = 12, 50, 5
    X = rng.standard_normal((n, r)) @ rng.standard_normal((r, d))
    P = O.calibrate(X)
    assert np.allclose(P.T @ P, np.eye(d), atol=1e-12)
    Y = X @ P
    assert np.max(np.abs(Y[:, r:])) < 1e-10 * np.max(np.abs(X))
    assert np.isclose(np.sum(Y ** 2), np.sum(X ** 2), rtol=1e-12)
    e = np.sum(Y ** 2, axis=0)
    assert np.all(np.diff(e[:r]) <= 1e-12 * e[0])
    # fewer samples than dims: still a full orthogonal P, the samples' span first
    X2 = rng.standard_normal((4, d))
    P2 = O.calibrate(X2)
    assert np.allclose(P2.T @ P2, np.eye(d), atol=1e-12)
    assert np.max(np.abs(X2 @ P2[:, 4:])) < 1e-10 * np.max(np.abs(X2))


def pin_calibrate_generator():
    """On the workload generator's own queries and keys (raw = Z diag(s) P^T, s decreasing), the
    calibrated P's leading r columns span the generator's leading r directions to within the
    sampling error of 16384 rows, and (Ky Fan: no r orthonormal directions capture more of the
    samples' energy than the top r right singular vectors) they capture at least as much energy
    as the generator's own columns."""
    from synth import make_qk_block, make_projection

    P64 = make_projection(2, 128)
    q, _ = make_qk_block(2, "calib_q", (0, 0), 8192, 128, 40.0, P64)
    k, _ = make_qk_block(2, "calib_k", (0, 0), 8192, 128, 40.0, P64)
    X = np.concatenate([q, k]).astype(np.float64)
    P = O.calibrate(X)
    for r in (16, 32, 64, 96):
        M = P64[:, :r].T @ P[:, :r]
        assert np.sum(M ** 2) / r > 0.99, r
        assert np.sum((X @ P[:, :r]) ** 2) >= np.sum((X @ P64[:, :r]) ** 2), r


PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_")}
