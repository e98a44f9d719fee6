"""GPU parity of the fused aqua_decode_step (append + select + decode in one launch)."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import (DEV, assert_close, check_mass_update, kp_token_major, mass_tol, new_cache,
                      oracle_decode, unpack_mask)
from oracle import aqua_oracle as O
from synth import config, make_decode_inputs, storage_to_f64

pytestmark = pytest.mark.gpu


def _step(inp, c, T, T_cap=None, mass=None, d_store=None, d_sel=None):
    """Cache holds tokens [0, T-1); the step appends token T-1 and attends [0, T)."""
    B, Hq, Hkv, d, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["k"]
    d_store = d_store or c.get("d_store", d)
    d_sel = d_sel or c.get("d_sel", d)
    T_cap = T_cap or ((T + 63) // 64 * 64)
    kp, v = new_cache(B, Hkv, d, d_store, T_cap, c["dtype"])
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    if T > 1:
        aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                             inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
    ws = torch.zeros(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_decode_step(cache, Hq, inp["q"].to(DEV), inp["k"][:, :, T - 1].contiguous().to(DEV),
                        inp["v"][:, :, T - 1].contiguous().to(DEV), P, d_sel, k,
                        1 / math.sqrt(d), out, ws, mass=mass, q_proj_out=qp, mask_out=mask)
    torch.cuda.synchronize()
    assert cache.len == T
    return dict(out=out, qp=qp, mask=mask, kp=kp, v=v, ws=ws, cache=cache, P=P)


@pytest.mark.parametrize("B,Hq,Hkv,T,k,d,dtype", [
    (2, 8, 2, 3000, 96, 128, "bf16"),
    (2, 8, 2, 2049, 96, 128, "bf16"),   # the new token opens a new split
    (1, 8, 2, 2048, 64, 128, "bf16"),   # the new token closes a split
    (1, 8, 2, 1, 96, 128, "bf16"),      # empty cache: the new token alone
    (2, 4, 4, 700, 48, 128, "bf16"),    # G = 1
    (1, 16, 2, 1000, 32, 128, "bf16"),  # G = 8
    (1, 4, 2, 1500, 100, 128, "f32"),
    (1, 1, 1, 256, 48, 64, "f32"),      # the tiny fp32 shape
])
def test_step_matches_oracle(B, Hq, Hkv, T, k, d, dtype):
    c = config(2 if dtype == "bf16" else 1, B=B, Hq=Hq, Hkv=Hkv, T=T, k=k, d=d, d_store=d,
               d_sel=d, dtype=dtype)
    inp = make_decode_inputs(c)
    r = _step(inp, c, T)
    m = unpack_mask(r["mask"], d)
    assert np.array_equal(m, O.select(r["qp"].cpu().double().numpy(), d, k))
    ref = oracle_decode(inp, c, m)
    assert_close(r["out"].cpu().double().numpy(), ref, dtype, "decode step")
    # the new token's K' and V are in the cache
    P64 = storage_to_f64(inp["P"])
    kn = O.project_keys_stored(storage_to_f64(inp["k"][:, :, T - 1]), P64, dtype, d)
    got = storage_to_f64(r["kp"])[:, :, :, T - 1]
    ulp = np.abs(kn) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)
    acc = d * 2.0 ** -24 * (np.abs(storage_to_f64(inp["k"][:, :, T - 1])) @ np.abs(P64))
    assert np.all(np.abs(got - kn) <= ulp + acc)
    assert np.array_equal(storage_to_f64(r["v"])[:, :, T - 1], storage_to_f64(inp["v"][:, :, T - 1]))


@pytest.mark.parametrize("T", [5000, 4096, 1500])
def test_step_equals_separate_calls(T):
    """q', masks and the cache are bit-identical to project + select + decode; outputs agree to
    fp32 summation order (split-T kernel, T > 4096), or bit for bit (short kernel: the new token
    takes its place in the same sums)."""
    c = config(2, B=4, Hq=32, Hkv=8, T=T)
    inp = make_decode_inputs(c)
    T, d, k, B, Hq = c["T"], c["d"], c["k"], c["B"], c["Hq"]
    r = _step(inp, c, T)
    kp, v = new_cache(B, c["Hkv"], d, d, r["kp"].shape[-1], "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = r["P"]
    aq.aqua_project_keys(cache, inp["k"].to(DEV), inp["v"].to(DEV), P, T)
    qp = torch.empty(B * Hq, d, device=DEV)
    mask = torch.empty(B * Hq, d // 32, dtype=torch.int32, device=DEV)
    aq.aqua_select_dims(inp["q"].reshape(B * Hq, d).to(DEV), P, d, k, qp, mask)
    ws = torch.zeros_like(r["ws"])
    out = torch.empty_like(r["out"])
    aq.aqua_decode(cache, Hq, qp, mask, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    assert torch.equal(qp.reshape(B, Hq, d), r["qp"])
    assert torch.equal(mask.reshape(B, Hq, d // 32), r["mask"])
    assert torch.equal(kp[..., :T], r["kp"][..., :T])
    assert torch.equal(v[:, :, :T], r["v"][:, :, :T])
    if T <= 4096:
        assert torch.equal(out, r["out"])
    else:
        assert torch.allclose(out, r["out"], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("T0", [2045, 4093])
def test_step_sequence_appends(T0):
    """Several steps in a row on one cache and workspace: each appends and attends correctly
    (across a 256-token chunk boundary of the short kernel, and across the switch from the
    short kernel to the split-T kernel after 4096 tokens)."""
    c = config(2, B=2, Hq=8, Hkv=2, T=T0 + 8)
    inp = make_decode_inputs(c)
    B, Hq, d, k = c["B"], c["Hq"], c["d"], c["k"]
    kp, v = new_cache(B, c["Hkv"], d, d, (T0 + 8 + 63) // 64 * 64, "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T0].contiguous().to(DEV),
                         inp["v"][:, :, :T0].contiguous().to(DEV), P, T0)
    ws = torch.zeros(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    q = inp["q"].to(DEV)
    for t in range(T0, T0 + 6):
        out = torch.full((B, Hq, d), float("nan"), device=DEV)
        mask = torch.empty(B, Hq, d // 32, dtype=torch.int32, device=DEV)
        aq.aqua_decode_step(cache, Hq, q, inp["k"][:, :, t].contiguous().to(DEV),
                            inp["v"][:, :, t].contiguous().to(DEV), P, d, k, 1 / math.sqrt(d),
                            out, ws, mask_out=mask)
        torch.cuda.synchronize()
        assert cache.len == t + 1
        m = unpack_mask(mask, d)
        ref = oracle_decode(inp, c, m, length=t + 1)
        assert_close(out.cpu().double().numpy(), ref, "bf16", f"step at {t}")


@pytest.mark.parametrize("T,T_cap", [(1280, 1280), (9000, 9024)])
def test_step_mass_mode(T, T_cap):
    """Mass mode of the fused step (short kernel at 1280 tokens, split-T past 4096): every token's
    mass, the new one's included, grows by the group's summed weight, per element within the
    derived relative bound (fp64 weights from the GPU's own q' and K')."""
    c = config(2, B=1, Hq=8, Hkv=2, T=T, d_store=96, d_sel=96, k=64)
    inp = make_decode_inputs(c)
    mass0 = torch.rand(c["B"], c["Hkv"], T_cap, device=DEV)
    mass = mass0.clone()
    r = _step(inp, c, c["T"], T_cap=T_cap, mass=mass)
    m = unpack_mask(r["mask"], c["d"])
    assert np.array_equal(m, O.select(r["qp"].cpu().double().numpy(), 96, 64))
    qp = r["qp"].cpu().double().numpy()
    G = c["Hq"] // c["Hkv"]
    scale = 1 / math.sqrt(c["d"])
    for g in range(c["Hkv"]):
        Kp = kp_token_major(r["kp"], 0, g, T)
        V = storage_to_f64(inp["v"][0, g])
        hs = slice(g * G, (g + 1) * G)
        add = O.h2o_seed_mass(qp[0, hs], m[0, hs], Kp, V, scale)
        tol = mass_tol(qp[0, hs], m[0, hs], Kp, scale, 64)
        check_mass_update(mass0[0, g, :T].cpu().numpy(), mass[0, g, :T].cpu().numpy(), add, tol,
                          f"group {g}")
        assert torch.equal(mass[0, g, T:], mass0[0, g, T:])


@pytest.mark.parametrize("k", [96, 32])
def test_step_long_context_sampled(k):
    """B=1, T=131072 (32 splits per KV group; the new token lands in the last one), with a spare
    capacity of 256 tokens; every mask checked, sampled heads against the oracle."""
    c = config(3, k=k)
    T, d = c["T"], c["d"]
    inp = make_decode_inputs(c, workers=8)
    r = _step(inp, c, T, T_cap=T + 256)
    m = unpack_mask(r["mask"], d)
    assert np.array_equal(m, O.select(r["qp"].cpu().double().numpy(), d, k))
    heads = [(0, 0), (0, 13), (0, 31)]
    ref = oracle_decode(inp, c, m, heads=heads)
    got = r["out"].cpu().double().numpy()
    for b, h in heads:
        assert_close(got[b, h], ref[b, h], "bf16", f"k={k} head {h}")


def test_short_steps_graph_replay():
    """Six aqua_decode_step calls at short lengths (the short-context kernel: 1500 tokens and up,
    24 workgroups), then an aqua_decode over the result, captured in one HIP graph: three replays
    from a restored cache give the bits of the same calls run eagerly, with the eager calls on the
    same workspace (other epochs in its counters) run between the replays."""
    c = config(2, B=2, Hq=8, Hkv=2, T=1506)
    inp = make_decode_inputs(c)
    B, Hq, Hkv, d, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["k"]
    T0, n = 1500, 6
    kp, v = new_cache(B, Hkv, d, d, (T0 + n + 63) // 64 * 64, "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T0].contiguous().to(DEV),
                         inp["v"][:, :, :T0].contiguous().to(DEV), P, T0)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    q = inp["q"].to(DEV)
    kn = [inp["k"][:, :, t].contiguous().to(DEV) for t in range(T0, T0 + n)]
    vn = [inp["v"][:, :, t].contiguous().to(DEV) for t in range(T0, T0 + n)]
    outs = [torch.empty(B, Hq, d, device=DEV) for _ in range(n + 1)]
    qp = torch.empty(B, Hq, d, device=DEV)
    mask = torch.empty(B, Hq, d // 32, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    start = (kp.clone(), v.clone())

    def restore():
        kp.copy_(start[0])
        v.copy_(start[1])
        for o in outs:
            o.fill_(float("nan"))
        cache.len = T0

    def calls():
        for i in range(n):
            aq.aqua_decode_step(cache, Hq, q, kn[i], vn[i], P, d, k, scale, outs[i], ws,
                                q_proj_out=qp, mask_out=mask)
        aq.aqua_decode(cache, Hq, qp, mask, scale, outs[n], ws)

    def snapshot():  # bit patterns: the cache's unwritten columns hold NaN
        ts = [o for o in outs] + [qp, mask, kp, v]
        return [t.view(torch.int16 if t.element_size() == 2 else torch.int32).clone() for t in ts]

    restore()
    calls()
    torch.cuda.synchronize()
    ref = snapshot()
    assert all(torch.isfinite(o).all() for o in outs)

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(graph, stream=s_cap):
            calls()
    torch.cuda.synchronize()
    for it in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (got, want) in enumerate(zip(snapshot(), ref)):
            assert torch.equal(got, want), f"replay {it}: tensor {j} differs from the eager calls"
        restore()
        calls()
        torch.cuda.synchronize()
        for j, (got, want) in enumerate(zip(snapshot(), ref)):
            assert torch.equal(got, want), f"eager calls after replay {it}: tensor {j} differs"
