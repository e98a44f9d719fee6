"""GPU parity of aqua_decode (with selection and key projection in front) against the oracle."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import (DEV, assert_close, check_mass_update, kp_token_major, mass_tol,
                      oracle_decode, rel_l2, run_decode, unpack_mask)
from oracle import aqua_oracle as O
from synth import config, make_decode_inputs, storage_to_f64

pytestmark = pytest.mark.gpu


def _check_masks(r, c, d_sel=None, k=None):
    d = c["d"]
    m = unpack_mask(r["mask"], d)
    qp = r["qp"].cpu().double().numpy()
    assert np.array_equal(m, O.select(qp, d_sel or c.get("d_sel", d), k or c["k"]))
    return m


def test_tiny_decode_f32():
    c = config(1)
    inp = make_decode_inputs(c)
    r = run_decode(inp, c)
    m = _check_masks(r, c)
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "f32", "tiny decode")


@pytest.mark.parametrize("Hq,Hkv,T,k,d", [
    (8, 2, 3000, 96, 128),     # G=4, two splits, ragged tail
    (4, 4, 2049, 64, 128),     # G=1
    (8, 4, 777, 128, 128),     # G=2, k = d
    (16, 2, 1500, 32, 128),    # G=8
    (8, 2, 1, 96, 128),        # a single token
    (4, 1, 513, 40, 64),       # d = 64
    # past 4096 tokens the split-T kernel runs (the cases above take the short-context one)
    (8, 2, 5000, 96, 128),     # G=4
    (4, 4, 4097, 64, 128),     # G=1
    (8, 4, 4200, 128, 128),    # G=2, k = d
    (16, 2, 4500, 32, 128),    # G=8
    (4, 1, 4300, 40, 64),      # d = 64
    # past 16 splits per group the merge takes two levels (runs of 8 splits; the last run ragged)
    # (B2 x 2 groups is a small grid: 4-wavefront workgroups, splits of 2048)
    (8, 2, 40000, 96, 128),    # G=4: 20 splits of 2048
    (8, 2, 70000, 96, 128),    # G=4: 35 splits of 2048
    (16, 2, 20000, 32, 128),   # G=8: 20 splits of 1024
])
def test_decode_bf16_shapes(Hq, Hkv, T, k, d):
    c = config(2, B=2, Hq=Hq, Hkv=Hkv, T=T, k=k, d=d, d_store=d, d_sel=d)
    inp = make_decode_inputs(c)
    r = run_decode(inp, c)
    m = _check_masks(r, c)
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "bf16", f"decode {Hq},{Hkv},{T}")


@pytest.mark.parametrize("T,far", [(3000, "early"), (3000, "late"), (9000, "early"),
                                   (9000, "late"), (40000, "early")])
def test_decode_far_apart_maxima(T, far):
    """Partials whose maxima lie ~24 log2 units apart: every query gets a common component 6u
    (u a seeded unit vector) and the keys of one half of the context are -33u, so that half's
    scores sit near -22 (log2 units) against ~2 elsewhere.  The merge of the splits (or of the
    short kernel's 256-token workgroups) must weigh the far half by ~2^-24, not drop or
    overflow it."""
    c = config(2, B=2, Hq=8, Hkv=2, T=T, k=96)
    inp = make_decode_inputs(c)
    u = np.random.default_rng(2025).standard_normal(c["d"])
    u = torch.from_numpy(u / np.linalg.norm(u))
    dt = inp["q"].dtype
    inp["q"] = (inp["q"].double() + 6.0 * u).to(dt)
    k = inp["k"].double()
    half = slice(0, T // 2) if far == "early" else slice(T // 2, T)
    k[:, :, half] = -33.0 * u
    inp["k"] = k.to(dt)
    r = run_decode(inp, c)
    m = _check_masks(r, c)
    # the two halves' maxima are far apart (oracle arithmetic, head 0)
    P64 = storage_to_f64(inp["P"])
    Kp = O.project_keys_stored(storage_to_f64(inp["k"][0, 0]), P64, c["dtype"], c["d"])
    qp = O.project(storage_to_f64(inp["q"][0, 0]), P64)
    sc = (np.where(m[0, 0], qp, 0) @ Kp.T) / math.sqrt(c["d"]) / math.log(2)
    far_max = sc[half].max()
    near_max = np.delete(sc, np.arange(T)[half]).max()
    assert near_max - far_max > 16
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "bf16", f"far maxima {T},{far}")


@pytest.mark.parametrize("T,d_store,k", [
    (3000, 96, 64),    # short-context kernel
    (3000, 64, 48),
    (9000, 96, 64),    # split-T kernel
    (9000, 64, 48),
    (70000, 64, 48),   # two-level merge (35 splits of 2048)
])
def test_decode_memory_cut(T, d_store, k):
    """AQUA-Memory's static cut at the decode shape: only K' dims [0, d_store) are stored and each
    query keeps its top-k of those; V is stored whole."""
    c = config(2, B=2, Hq=8, Hkv=2, T=T, k=k, d_store=d_store, d_sel=d_store)
    inp = make_decode_inputs(c)
    r = run_decode(inp, c)
    assert r["kp"].shape[2] == d_store
    m = _check_masks(r, c)
    assert not m[..., d_store:].any()
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "bf16", f"memory cut {T},{d_store},{k}")


@pytest.mark.parametrize("T,k", [(3000, 96), (9000, 32)])
def test_decode_static_first_k_mask(T, k):
    """aqua_decode takes any mask: the first-k slicing baseline (dims [0, k) for every query)
    against the oracle on the same mask."""
    c = config(2, B=2, Hq=8, Hkv=2, T=T, k=k)
    inp = make_decode_inputs(c)
    B, Hq, Hkv, d = c["B"], c["Hq"], c["Hkv"], c["d"]
    r = run_decode(inp, c)  # builds the cache and q'; its own masks are not used below
    m = np.zeros((B, Hq, d), bool)
    m[..., :k] = True
    words = np.packbits(m.reshape(B * Hq, d), axis=-1, bitorder="little").view(np.int32)
    mask = torch.from_numpy(words.copy()).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = torch.zeros_like(r["ws"])
    aq.aqua_decode(r["cache"], Hq, r["qp"].reshape(B * Hq, d), mask, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    ref = oracle_decode(inp, c, m)
    assert_close(out.cpu().double().numpy(), ref, "bf16", f"first-{k} mask, T={T}")


@pytest.mark.parametrize("length", [1, 63, 255, 256, 257, 511, 512, 2047, 2048, 2049, 4096, 4097,
                                    4100])
def test_decode_ragged_lengths_f32(length):
    """fp32 storage: tight tolerance across split and wavefront boundaries; T_cap > len."""
    c = config(1, B=1, Hq=4, Hkv=2, d=128, T=length, k=100, d_store=128, d_sel=128)
    inp = make_decode_inputs(c)
    r = run_decode(inp, c, T_cap=4160)
    m = _check_masks(r, c)
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "f32", f"len {length}")


def test_decode_deterministic_and_reusable_workspace():
    c = config(2, B=2, Hq=8, Hkv=2, T=5000)
    inp = make_decode_inputs(c)
    r = run_decode(inp, c)
    outs = []
    for _ in range(3):
        out = torch.full_like(r["out"], float("nan"))
        aq.aqua_decode(r["cache"], c["Hq"], r["qp"], r["mask"], 1 / math.sqrt(c["d"]), out,
                       r["ws"])
        outs.append(out)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, r["out"])


def test_decode_workspace_reuse_across_inputs():
    """Calls that share one workspace but attend different queries and contexts, alternating:
    each output must match a fresh single call (no stale partials, counters reset)."""
    c = config(2, B=2, Hq=8, Hkv=2, T=6000)
    runs = []
    for seed_cfg in (2, 4):
        cc = dict(c, id=seed_cfg)
        inp = make_decode_inputs(cc)
        runs.append(run_decode(inp, cc))
    ws = torch.zeros_like(runs[0]["ws"])
    scale = 1 / math.sqrt(c["d"])
    for it in range(6):
        r = runs[it % 2]
        out = torch.full_like(r["out"], float("nan"))
        aq.aqua_decode(r["cache"], c["Hq"], r["qp"], r["mask"], scale, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, r["out"]), f"call {it}"


@pytest.fixture(scope="module")
def long_inputs():
    return make_decode_inputs(config(3))


@pytest.mark.parametrize("k", [128, 96, 64, 32])
def test_decode_long_context_sampled(k, long_inputs):
    """B=1, T=131072 (many splits per group), every k of the sweep; sampled heads."""
    c = config(3, k=k)
    inp = long_inputs
    r = run_decode(inp, c, k=k)
    m = _check_masks(r, c, k=k)
    heads = [(0, 0), (0, 5), (0, 22), (0, 31)]
    ref = oracle_decode(inp, c, m, heads=heads)
    got = r["out"].cpu().double().numpy()
    for b, h in heads:
        assert_close(got[b, h], ref[b, h], "bf16", f"k={k} head {h}")


def check_mass_mode(r, inp, c, mass0, mass):
    """Mass mode: every token's mass grew by the group's summed softmax weight, per element within
    the weights' derived relative bound (gpu_util.mass_tol), the fp64 weights computed from the
    GPU's own q' and K'; the sum of the additions is G; tokens past len are untouched."""
    B, Hq, Hkv, d, T, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"], c["k"]
    G = Hq // Hkv
    scale = 1 / math.sqrt(d)
    m = unpack_mask(r["mask"], d)
    qp = r["qp"].cpu().double().numpy()
    before = mass0.cpu().double().numpy()
    after = mass.cpu().double().numpy()
    for b in range(B):
        for g in range(Hkv):
            Kp = kp_token_major(r["kp"], b, g, T)
            V = storage_to_f64(inp["v"][b, g, :T])
            hs = slice(g * G, (g + 1) * G)
            add = O.h2o_seed_mass(qp[b, hs], m[b, hs], Kp, V, scale)
            tol = mass_tol(qp[b, hs], m[b, hs], Kp, scale, k)
            check_mass_update(before[b, g, :T], after[b, g, :T], add, tol, f"group {(b, g)}")
            assert abs((after[b, g, :T] - before[b, g, :T]).sum() - G) < 1e-3
            assert np.array_equal(after[b, g, T:], before[b, g, T:])


@pytest.mark.parametrize("T", [3000, 40000, 70000])
def test_decode_mass_accumulation(T):
    """Mass mode: mass[t] grows by the sum over the group's heads of the softmax weights (short
    kernel at 3000 tokens; split-T kernel with the two-level merge at 40000 and 70000)."""
    c = config(2, B=2, Hq=8, Hkv=2, T=T, d_store=96, d_sel=96, k=64)
    inp = make_decode_inputs(c)
    T_cap = (T + 8 + 63) // 64 * 64
    mass0 = torch.rand(c["B"], c["Hkv"], T_cap, device=DEV)
    mass = mass0.clone()
    r = run_decode(inp, c, T_cap=T_cap, mass=mass)
    _check_masks(r, c)
    check_mass_mode(r, inp, c, mass0, mass)


def test_decode_mass_eight_wave_d64():
    """Mass mode and d = 64 on the 8-wavefront layout (16 groups x 16 full 4096-token splits:
    one 512-thread workgroup per CU of a 256-CU device), against the oracle on every head."""
    c = config(2, B=2, Hq=32, Hkv=8, T=65536, d=64, d_store=64, d_sel=64, k=40)
    inp = make_decode_inputs(c, workers=16)
    T_cap = c["T"] + 256
    mass0 = torch.rand(c["B"], c["Hkv"], T_cap, device=DEV)
    mass = mass0.clone()
    r = run_decode(inp, c, T_cap=T_cap, mass=mass)
    m = _check_masks(r, c)
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "bf16", "d=64, 8-wave")
    check_mass_mode(r, inp, c, mass0, mass)


@pytest.mark.parametrize("B,Hq,Hkv,T", [
    (4, 32, 8, 16384),   # 32 groups x 8 full 2048-token splits: the 8-wavefront layout
    (2, 8, 2, 9000),     # 4 groups: the 4-wavefront layout (1024-token splits)
])
def test_decode_f32_group4_layouts(B, Hq, Hkv, T):
    """fp32 storage at G = 4 on the split-T kernel in both layouts, every head against the oracle
    within the fp32 tolerance."""
    c = config(1, B=B, Hq=Hq, Hkv=Hkv, d=128, T=T, k=96, d_store=128, d_sel=128)
    inp = make_decode_inputs(c, workers=16)
    r = run_decode(inp, c)
    m = _check_masks(r, c)
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, "f32", f"f32 G=4 {B},{T}")
