"""GPU parity of H2O decoding over a compact AQUA-Memory cache against the oracle.

Per step, following the parity protocol for H2O: the GPU's slot set must equal the oracle's
heavy + recent set computed from the GPU's own (fp32) mass; the masks must equal the oracle's
selection of the GPU's q'; the output must match the fp64 attention over that set; and the GPU's
mass after the step must equal its mass before plus the fp64 softmax weights.

Mass tolerance (no figure is given for it, so it is derived from the arithmetic: gpu_util's
mass_tol).  The oracle's weights are computed from the GPU's own q' and K' (their roundings are
checked by the selection and key-projection tests: one bf16 ulp of K' alone moves a weight by
~1e-4), so the GPU's weights differ only by the fp32 score sum and the exp2/divide roundings.  The
bound is computed from the data at every check.

Both step forms are checked this way: the four calls (victim, slot append, selection, mass-mode
decode) and the one launch aqua_h2o_step.  The starting state comes from aqua_h2o_init, whose
slot set is checked against the oracle's heavy set of the GPU's seeding mass, bit for bit."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from sparse_dimension_attention_amd.h2o import H2OCache
from gpu_util import (DEV, BF16_MAXABS, BF16_RELL2, F32_TOL, mass_tol, new_cache, rel_l2,
                      unpack_mask)
from oracle import aqua_oracle as O
from synth import config, make_h2o_inputs, storage_to_f64

pytestmark = pytest.mark.gpu

_mass_tol = mass_tol


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


def _run(c, fused=False):
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
                P, t_new, c["d_sel"], c["k"], scale, out, qp, mask, fused=fused)
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


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_h2o_step_instances(dtype, d, G):
    """The one-launch step in every compiled form (storage dtype x d x G): 128 slots (96 heavy,
    32 recent) over a 400-token context, 3 steps, every step against the oracle."""
    _run(config(5, B=1, Hq=2 * G, Hkv=2, d=d, d_store=d, d_sel=d, k=3 * d // 4, T=400,
                heavy=96, recent=32, steps=3, dtype=dtype), fused=True)


def _draw_h2o_shapes(n, seed=20261206):
    """H2O shapes from a fixed seed: batch 1-2, 1-3 KV heads, G = 1/2/4/8, d 64 or 128, any
    d_store, d_sel and k below it, bf16 or fp32, a compact cache of 64-1024 slots split into a
    heavy part and a recent window (both non-empty), contexts from the slot count up to 9000
    tokens (so the seeding decode runs on either decode kernel), 4-12 steps."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 4))
        d_store = d if rng.random() < 0.33 else int(rng.integers(1, d + 1))
        d_sel = d_store if rng.random() < 0.5 else int(rng.integers(1, d_store + 1))
        n_slots = 64 * int(rng.integers(1, 17))
        recent = int(rng.integers(1, n_slots))
        shapes.append(dict(B=int(rng.integers(1, 3)), Hq=G * Hkv, Hkv=Hkv, d=d, d_store=d_store,
                           d_sel=d_sel, k=int(rng.integers(1, d_sel + 1)),
                           T=int(rng.integers(n_slots, 9001)), heavy=n_slots - recent,
                           recent=recent, steps=int(rng.integers(4, 13)),
                           dtype="bf16" if rng.random() < 0.6 else "f32"))
    return shapes


H2O_SHAPES = _draw_h2o_shapes(8)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("over", H2O_SHAPES, ids=[
    f"{o['dtype']}-B{o['B']}-Hq{o['Hq']}-Hkv{o['Hkv']}-d{o['d']}-ds{o['d_store']}-dsel{o['d_sel']}"
    f"-k{o['k']}-T{o['T']}-h{o['heavy']}-r{o['recent']}-s{o['steps']}" for o in H2O_SHAPES])
def test_h2o_shape_sweep(over, fused):
    """Drawn shapes through the whole H2O sequence (seeding decode in mass mode, aqua_h2o_init,
    then the steps as four calls or as the one launch), checked against the oracle at every step
    as in the workload test above."""
    _run(config(5, **over), fused=fused)


@pytest.mark.parametrize("fused", [False, True])
def test_h2o_llama8b_t32768_64_steps(fused):
    """The heavy-hitter workload: 32768-token context, 1024 heavy + 256 recent slots, AQUA-Memory
    (96 stored dims, top-64 of them), 64 steps; as four calls per step and as the one launch
    aqua_h2o_step (the benchmarked form), each checked against the oracle at every step."""
    _run(config(5), fused=fused)


def test_h2o_small_fused_every_step_evicts():
    """The one-launch step against the oracle where every step evicts (fp32 storage, G = 4) and
    with G = 8 in bf16."""
    _run(config(5, T=320, heavy=40, recent=24, steps=48, dtype="f32"), fused=True)
    _run(config(5, Hq=16, Hkv=2, T=700, heavy=96, recent=32, steps=40), fused=True)


@pytest.mark.parametrize("T,heavy,recent,ties", [
    (32768, 1024, 256, False),   # the heavy-hitter workload's shape
    (5000, 668, 100, True),      # masses from a 5-value set: ties ranked by position
    (2048, 1984, 64, True),      # every older position is a heavy hitter
    (640, 0, 64, False),         # recent window only
    (2000, 64, 0, True),         # no recent window
])
def test_h2o_init_matches_oracle(T, heavy, recent, ties):
    """aqua_h2o_init: each (b, g)'s slot positions are the oracle's heavy set of the same (fp32)
    mass, in ascending order, followed by the recent window, bit for bit; every slot's K' column,
    V row and mass are the full cache's at that position, bit for bit."""
    B, Hkv, d, d_store = 2, 4, 128, 96
    T_cap = (T + 63) // 64 * 64
    g = torch.Generator(device="cpu").manual_seed(T + heavy)
    kp = torch.randn(B, Hkv, d_store, T_cap, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, Hkv, T_cap, d, generator=g).to(torch.bfloat16).to(DEV)
    if ties:
        vals = torch.tensor([0.0, 1e-3, 2e-3, 0.5, 3e-7])
        mass = vals[torch.randint(0, 5, (B, Hkv, T_cap), generator=g)]
    else:
        mass = torch.rand(B, Hkv, T_cap, generator=g) ** 4
    mass = mass.float().to(DEV)
    n = heavy + recent
    kc = torch.full((B, Hkv, d_store, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((B, Hkv, n, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    mc = torch.full((B, Hkv, n), float("nan"), device=DEV)
    pos = torch.full((B, Hkv, n), -7, dtype=torch.int32, device=DEV)
    aq.aqua_h2o_init(aq.make_cache(kp, v, T), mass, heavy, recent, aq.make_cache(kc, vc, n), mc,
                     pos)
    torch.cuda.synchronize()
    pos_np = pos.cpu().numpy().astype(np.int64)
    m64 = mass.cpu().double().numpy()
    for b in range(B):
        for gg in range(Hkv):
            H = O.h2o_heavy_set(m64[b, gg, :T], T - 1, heavy, recent) if heavy else \
                np.zeros(0, np.int64)
            want = np.concatenate([H, np.arange(T - recent, T)])
            assert np.array_equal(pos_np[b, gg], want), f"group {(b, gg)}"
            idx = torch.from_numpy(want).to(DEV)
            assert torch.equal(kc[b, gg], kp[b, gg][:, idx])
            assert torch.equal(vc[b, gg], v[b, gg][idx])
            assert torch.equal(mc[b, gg], mass[b, gg][idx])


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


@pytest.mark.parametrize("fused", [True, False])
def test_h2o_steps_graph_replay(fused):
    """H2O steps captured in a HIP graph and replayed from a restored starting state give the bits
    of the same steps run eagerly: every replay runs with the epochs taken at capture, and the
    library needs no clearing between replays.  Eager steps on the same workspace (other epochs
    in its counters) run between the replays.  The compact cache holds 128 slots, so every
    attention launch is the short-context kernel (one launch per step, or the four calls)."""
    c = config(5, Hq=16, Hkv=2, T=700, heavy=96, recent=32, steps=12)
    inp = make_h2o_inputs(c)
    B, Hq, d, T, S = c["B"], c["Hq"], c["d"], c["T"], c["steps"]
    st, _, _, _, P, _ = _seed(inp, c)
    st.workspace(Hq)
    scale = 1 / math.sqrt(d)
    qs, ks, vs = (inp[x].to(DEV) for x in ("q_steps", "k_steps", "v_steps"))
    out = torch.empty(B, Hq, d, device=DEV)
    qp = torch.empty(B, Hq, d, device=DEV)
    mask = torch.empty(B, Hq, d // 32, dtype=torch.int32, device=DEV)
    state = (st.kp, st.v, st.slot_pos, st.mass)
    start = [t.clone() for t in state]

    def restore():
        for dst, src in zip(state, start):
            dst.copy_(src)
        for t in (out, qp):
            t.fill_(float("nan"))
        mask.fill_(-1)
        st.victim.fill_(-7)

    def steps():
        for s in range(S):
            st.step(qs[s], ks[s], vs[s], P, T + s, c["d_sel"], c["k"], scale, out, qp, mask,
                    fused=fused)

    def snapshot():
        return [t.clone() for t in (out, qp, mask, st.victim, *state)]

    restore()
    steps()
    torch.cuda.synchronize()
    ref = snapshot()
    assert all(torch.isfinite(t).all() for t in (ref[0], ref[1]))

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(graph, stream=s_cap):
            steps()
    torch.cuda.synchronize()
    names = ("out", "q_proj", "mask", "victim", "K'", "V", "slot_pos", "mass")
    for it in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, snapshot(), ref):
            assert torch.equal(got, want), f"replay {it}: {name} differs from the eager steps"
        restore()
        steps()
        torch.cuda.synchronize()
        for name, got, want in zip(names, snapshot(), ref):
            assert torch.equal(got, want), f"eager run after replay {it}: {name} differs"
