"""GPU parity of H2O decoding over a compact AQUA-Memory cache against the oracle.

Per step, following the parity protocol for H2O: the GPU's slot set must equal the oracle's
heavy + recent set computed from the GPU's own (fp32) mass; the masks must equal the oracle's
selection of the GPU's q'; the output must match the fp64 attention over that set; and the GPU's
mass after the step must equal its mass before plus the fp64 softmax weights.

Mass tolerance (no figure is given for it, so it is derived from the arithmetic).  The oracle's
weights are computed from the GPU's own q' and K' (their roundings are checked by the selection
and key-projection tests: one bf16 ulp of K' alone moves a weight by ~1e-4), so the GPU's
weights differ only by the fp32 score sum and the exp2/divide roundings: a score error
|ds| <= gamma_{n+2} * scale * sum_i |q'_i K'_i| (n = k terms; gamma_n = n u / (1 - n u),
u = 2^-24) moves p_t by a factor exp(ds_t - sum_u p_u ds_u), i.e. relative error <= 2 max|ds|;
the log2-domain subtraction s - max s, exp2, the division and the fp32 mass additions add a few
u more.  The bound is computed from the
data at every check."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from sparse_dimension_attention_amd.h2o import H2OCache
from gpu_util import DEV, BF16_MAXABS, BF16_RELL2, F32_TOL, new_cache, rel_l2, unpack_mask
from oracle import aqua_oracle as O
from synth import config, make_h2o_inputs, storage_to_f64

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _gamma(n):
    return n * U / (1 - n * U)


def _mass_tol(qp, m, Kp, scale, k):
    """Relative bound on the GPU's softmax weights: qp, m [G][d] (GPU q', masks), Kp [n][d_store]."""
    S = scale * float((np.abs(qp[:, :Kp.shape[1]] * m[:, :Kp.shape[1]]) @ np.abs(Kp).T).max())
    # 2 max|ds|; the log2-domain subtraction s - m (|s - m| <= 2 S log2 e) rounds once more
    return 2 * _gamma(k + 2) * S + 6 * U * S + 8 * U


def _seed(inp, c):
    """Full cache of the context, the seeding decode in mass mode, then the compact cache."""
    B, Hq, Hkv, d, T = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"]
    d_store, d_sel, k = c["d_store"], c["d_sel"], c["k"]
    T_cap = (T + 63) // 64 * 64
    kp, v = new_cache(B, Hkv, d, d_store, T_cap, c["dtype"])
    full = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(full, inp["k"].to(DEV), inp["v"].to(DEV), P, T)
    qp = torch.empty(B, Hq, d, device=DEV)
    mask = torch.empty(B, Hq, d // 32, dtype=torch.int32, device=DEV)
    aq.aqua_select_dims(inp["q_seed"].to(DEV), P, d_sel, k, qp, mask)
    mass = torch.zeros(B, Hkv, T_cap, device=DEV)
    ws = torch.zeros(aq.aqua_decode_workspace(full, Hq), dtype=torch.uint8, device=DEV)
    out = torch.empty(B, Hq, d, device=DEV)
    aq.aqua_decode(full, Hq, qp, mask, 1 / math.sqrt(d), out, ws, mass=mass)
    st = H2OCache.from_full(kp, v, mass, T, c["heavy"], c["recent"])
    torch.cuda.synchronize()
    return st, qp, mask, mass[:, :, :T], P, kp


def _run(c):
    inp = make_h2o_inputs(c)
    B, Hq, Hkv, d, T, S = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"], c["steps"]
    G = Hq // Hkv
    scale = 1 / math.sqrt(d)
    st, qp_seed, mask_seed, mass_seed, P, kp_full = _seed(inp, c)
    P64 = storage_to_f64(inp["P"])

    # oracle state per group: projected keys of context + steps, values, mass by position
    Kp, KpG, V, M = {}, {}, {}, {}  # oracle K', the GPU's K', values, the GPU's mass
    m_seed = unpack_mask(mask_seed, d)
    assert np.array_equal(m_seed.reshape(-1, d),
                          O.select(qp_seed.cpu().double().numpy().reshape(-1, d), c["d_sel"],
                                   c["k"]))
    gm = mass_seed.cpu().double().numpy()
    worst_mass = 0.0
    for b in range(B):
        for g in range(Hkv):
            kall = np.concatenate([storage_to_f64(inp["k"][b, g]),
                                   storage_to_f64(inp["k_steps"][:, b, g])])
            Kp[b, g] = O.project_keys_stored(kall, P64, c["dtype"], c["d_store"])
            V[b, g] = np.concatenate([storage_to_f64(inp["v"][b, g]),
                                      storage_to_f64(inp["v_steps"][:, b, g])])
            KpG[b, g] = np.zeros_like(Kp[b, g])
            KpG[b, g][:T] = kp_full[b, g, :, :T].T.cpu().double().numpy()
            hs = slice(g * G, (g + 1) * G)
            qs = qp_seed[b, hs].cpu().double().numpy()
            m64 = O.h2o_seed_mass(qs, m_seed[b, hs], KpG[b, g][:T], V[b, g][:T], scale)
            tol = _mass_tol(qs, m_seed[b, hs], KpG[b, g][:T], scale, c["k"])
            worst_mass = max(worst_mass, float(np.max(np.abs(gm[b, g] - m64) / m64)) / tol)
            M[b, g] = np.concatenate([gm[b, g], np.zeros(S)])  # the GPU's mass, by position
    assert worst_mass <= 1.0, f"seed mass error / bound {worst_mass}"

    # starting slot set = heavy set of the seed mass (oracle rule) + the recent window
    pos0 = st.slot_pos.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            want = np.concatenate([O.h2o_heavy_set(M[b, g], T - 1, c["heavy"], c["recent"]),
                                   np.arange(T - c["recent"], T)])
            assert np.array_equal(np.sort(pos0[b, g]), want)

    out = torch.empty(B, Hq, d, device=DEV)
    qp = torch.empty(B, Hq, d, device=DEV)
    mask = torch.empty(B, Hq, d // 32, dtype=torch.int32, device=DEV)
    refs, gots = [], []
    for s in range(S):
        t_new = T + s
        st.step(inp["q_steps"][s].to(DEV), inp["k_steps"][s].to(DEV), inp["v_steps"][s].to(DEV),
                P, t_new, c["d_sel"], c["k"], scale, out, qp, mask)
        torch.cuda.synchronize()
        pos = st.slot_pos.cpu().numpy()
        victim = st.victim.cpu().numpy()
        mass_g = st.mass.cpu().double().numpy()
        m_np = unpack_mask(mask, d)
        qp_np = qp.cpu().double().numpy()
        assert np.array_equal(m_np.reshape(-1, d),
                              O.select(qp_np.reshape(-1, d), c["d_sel"], c["k"])), f"step {s}"
        qraw = storage_to_f64(inp["q_steps"][s])
        for b in range(B):
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                KpG[b, g][t_new] = st.kp[b, g, :, int(victim[b, g])].cpu().double().numpy()
                rest = (V[b, g], M[b, g][:t_new + 1], t_new, c["heavy"], c["recent"], scale)
                ref, _, A_set = O.h2o_step(O.project(qraw[b, hs], P64), m_np[b, hs], Kp[b, g],
                                           *rest)
                _, new_mass, A2 = O.h2o_step(qp_np[b, hs], m_np[b, hs], KpG[b, g], *rest)
                assert np.array_equal(A_set, A2)
                assert np.array_equal(np.sort(pos[b, g]), A_set), f"step {s} group {g}"
                assert pos[b, g, victim[b, g]] == t_new
                refs.append(ref)
                gots.append(out[b, hs].cpu().double().numpy())
                # the GPU's mass after the step = its mass before + the fp64 weights
                want = new_mass[pos[b, g]]
                tol = _mass_tol(qp_np[b, hs], m_np[b, hs], KpG[b, g][A_set], scale, c["k"])
                dm = np.abs(mass_g[b, g] - want)
                assert np.all(dm <= tol * want), (
                    f"step {s} group {g} mass rel {float(np.max(dm / want))} > {tol}")
                M[b, g][pos[b, g]] = mass_g[b, g]  # carry the GPU's mass forward
    got, ref = np.stack(gots), np.stack(refs)
    err = float(np.max(np.abs(got - ref)))
    if c["dtype"] == "f32":
        assert err < F32_TOL, err
    else:
        assert err < BF16_MAXABS and rel_l2(got, ref) < BF16_RELL2, (err, rel_l2(got, ref))
    return inp, st


def test_h2o_small_many_evictions_f32():
    """fp32 storage, 320-token context, 40 heavy + 24 recent slots, 48 steps: every step evicts."""
    _run(config(5, T=320, heavy=40, recent=24, steps=48, dtype="f32"))


def test_h2o_small_bf16_g8():
    c = config(5, Hq=16, Hkv=2, T=700, heavy=96, recent=32, steps=40)
    _run(c)


def test_h2o_llama8b_t32768_64_steps():
    """The heavy-hitter workload: 32768-token context, 1024 heavy + 256 recent slots, AQUA-Memory
    (96 stored dims, top-64 of them), 64 steps."""
    _run(config(5))


@pytest.mark.parametrize("over", [
    dict(T=320, heavy=40, recent=24, steps=48, dtype="f32"),   # every step evicts
    dict(Hq=16, Hkv=2, T=700, heavy=96, recent=32, steps=40),  # G = 8
    dict(Hq=8, Hkv=8, T=900, heavy=200, recent=56, steps=24),  # G = 1, 256 slots: one chunk
    dict(steps=16),                                            # the 32768-token workload
])
def test_h2o_fused_step_equals_separate_calls(over):
    """aqua_h2o_step against the four calls (victim, slot append, selection, mass-mode decode)
    from two copies of the same state: every output and every piece of state equal, bit for
    bit, after every step (the separate calls are checked against the oracle above)."""
    c = config(5, **over)
    inp = make_h2o_inputs(c)
    st, _, _, _, P, _ = _seed(inp, c)
    st2 = H2OCache(st.kp.clone(), st.v.clone(), st.slot_pos.clone(), st.mass.clone(), st.heavy,
                   st.recent)
    B, Hq, d = c["B"], c["Hq"], c["d"]
    bufs = [(torch.empty(B, Hq, d, device=DEV), torch.empty(B, Hq, d, device=DEV),
             torch.empty(B, Hq, d // 32, dtype=torch.int32, device=DEV)) for _ in range(2)]
    scale = 1 / math.sqrt(d)
    for s in range(c["steps"]):
        args = (inp["q_steps"][s].to(DEV), inp["k_steps"][s].to(DEV), inp["v_steps"][s].to(DEV),
                P, c["T"] + s, c["d_sel"], c["k"], scale)
        st.step(*args, *bufs[0])
        st2.step(*args, *bufs[1], fused=True)
        torch.cuda.synchronize()
        for name, x, y in (("out", bufs[0][0], bufs[1][0]), ("q'", bufs[0][1], bufs[1][1]),
                           ("mask", bufs[0][2], bufs[1][2]), ("victim", st.victim, st2.victim),
                           ("slot_pos", st.slot_pos, st2.slot_pos), ("mass", st.mass, st2.mass),
                           ("K'", st.kp, st2.kp), ("V", st.v, st2.v)):
            assert torch.equal(x, y), f"step {s}: {name} differs"
