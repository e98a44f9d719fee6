"""Seeded sweeps of shapes against the oracle: the fused decode step and the decode call, and
the chunked prefill.

The shapes are drawn once, from a fixed seed, over the ranges the C ABI accepts: batch 1-3, 1-3
KV heads, group sizes 1, 2, 4 and 8, d 64 or 128, any stored-dim cut d_store, any d_sel up to
it, any k up to d_sel, bf16 or fp32 storage, contexts from 1 to 12000 tokens on both sides of
the switch between the short-context and the split-T kernels, and a cache capacity 0-3 tiles
past the context.  Per shape: aqua_decode_step appends token T-1 to a cache of T-1 tokens and
decodes; its masks must be the oracle's selection of its q' (exactly k dims, all below d_sel,
ties to the lower index), its outputs the oracle's attention over the first T tokens (stored
inputs, fp64), the appended K' column the oracle's projection within the rounding bound, and
the appended V row the input.  aqua_decode then runs on the same cache with the step's q' and
masks and must give the same outputs (to fp32 summation order).

The prefill sweep draws batch 1-2, 1-2 KV heads, group sizes 1, 2, 4 and 8, a stored-dim cut
that is a multiple of 16 (the prefill's operand granularity), any d_sel and k below it, up to
1000 tokens split into 1-4 chunks of random lengths, and a padded capacity, plus one fixed shape
whose chunks alternate single queries and whole tiles; every row's mask and output is checked."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import DEV, assert_close, new_cache, oracle_decode, unpack_mask
from oracle import aqua_oracle as O
from synth import config, make_decode_inputs, make_prefill_inputs, storage_to_f64

pytestmark = pytest.mark.gpu


def _draw_shapes(n, seed=20261204):
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 4))
        # a third of the shapes store every dim; the rest cut at any point
        d_store = d if rng.random() < 0.33 else int(rng.integers(1, d + 1))
        d_sel = d_store if rng.random() < 0.5 else int(rng.integers(1, d_store + 1))
        k = int(rng.integers(1, d_sel + 1))
        # half below the switch to the split-T kernel (4096 tokens), half above
        T = int(np.exp(rng.uniform(0.0, np.log(4096)))) if i % 2 == 0 else \
            int(rng.integers(4097, 12001))
        T = max(T, 1)
        T_cap = (T + 63) // 64 * 64 + 64 * int(rng.integers(0, 4))
        shapes.append(dict(B=B, Hq=G * Hkv, Hkv=Hkv, d=d, d_store=d_store, d_sel=d_sel, k=k,
                           T=T, T_cap=T_cap, dtype=dtype))
    return shapes


SHAPES = _draw_shapes(20)


def _id(s):
    return (f"{s['dtype']}-B{s['B']}-Hq{s['Hq']}-Hkv{s['Hkv']}-d{s['d']}-ds{s['d_store']}"
            f"-dsel{s['d_sel']}-k{s['k']}-T{s['T']}-cap{s['T_cap']}")


@pytest.mark.parametrize("s", SHAPES, ids=[_id(s) for s in SHAPES])
def test_shape_sweep_step_and_decode(s):
    c = config(2 if s["d"] == 128 else 1, **{k: v for k, v in s.items() if k != "T_cap"})
    inp = make_decode_inputs(c)
    B, Hq, Hkv, d, T, k = s["B"], s["Hq"], s["Hkv"], s["d"], s["T"], s["k"]
    d_store, d_sel, dtype = s["d_store"], s["d_sel"], s["dtype"]
    kp, v = new_cache(B, Hkv, d, d_store, s["T_cap"], dtype)
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    if T > 1:
        aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                             inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
    # a workspace of random bytes: the counters carry epochs and need no clearing
    nws = aq.aqua_decode_workspace(cache, Hq)
    g = torch.Generator().manual_seed(T)
    ws = torch.randint(0, 256, (nws,), dtype=torch.uint8, generator=g).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    aq.aqua_decode_step(cache, Hq, inp["q"].to(DEV), inp["k"][:, :, T - 1].contiguous().to(DEV),
                        inp["v"][:, :, T - 1].contiguous().to(DEV), P, d_sel, k, scale, out, ws,
                        q_proj_out=qp, mask_out=mask)
    torch.cuda.synchronize()
    assert cache.len == T

    m = unpack_mask(mask, d)
    assert np.array_equal(m, O.select(qp.cpu().double().numpy(), d_sel, k))
    ref = oracle_decode(inp, c, m, d_store=d_store)
    assert_close(out.cpu().double().numpy(), ref, dtype, "step")

    # the appended token: K' dims below d_store within one rounding plus the fp32 sum's error
    P64 = storage_to_f64(inp["P"])
    kin = storage_to_f64(inp["k"][:, :, T - 1])
    kn = O.project_keys_stored(kin, P64, dtype, d_store)
    got = storage_to_f64(kp)[:, :, :, T - 1]
    ulp = np.abs(kn) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)
    acc = (d * 2.0 ** -24 * (np.abs(kin) @ np.abs(P64)))[..., :d_store]
    assert np.all(np.abs(got - kn) <= ulp + acc)
    assert np.array_equal(storage_to_f64(v)[:, :, T - 1], storage_to_f64(inp["v"][:, :, T - 1]))

    # the decode call on the same cache, q' and masks (the step's workspace, reused as it is)
    out2 = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp.reshape(B * Hq, d), mask.reshape(B * Hq, d // 32), scale, out2,
                   ws)
    torch.cuda.synchronize()
    assert torch.allclose(out2, out, rtol=1e-5, atol=1e-6), \
        float((out2 - out).abs().max())


def _draw_prefill_shapes(n, seed=20261205):
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3))
        B = int(rng.integers(1, 3))
        d_store = 16 * int(rng.integers(1, 9))
        d_sel = d_store if rng.random() < 0.5 else int(rng.integers(1, d_store + 1))
        k = int(rng.integers(1, d_sel + 1))
        T = int(rng.integers(1, 1001))
        nch = int(rng.integers(1, 5))
        cuts = sorted({int(x) for x in rng.integers(1, T, size=nch - 1)}) if T > 1 else []
        bounds = [0, *cuts, T]
        chunks = [b1 - b0 for b0, b1 in zip(bounds[:-1], bounds[1:])]
        T_cap = (T + 63) // 64 * 64 + 64 * int(rng.integers(0, 3))
        shapes.append(dict(B=B, Hq=G * Hkv, Hkv=Hkv, d_store=d_store, d_sel=d_sel, k=k, T=T,
                           chunks=chunks, T_cap=T_cap))
    return shapes


PREFILL_SHAPES = _draw_prefill_shapes(10) + [
    dict(B=1, Hq=4, Hkv=1, d_store=128, d_sel=128, k=96, T=131, chunks=[1, 64, 1, 64, 1],
         T_cap=192)]


def _pid(s):
    return (f"B{s['B']}-Hq{s['Hq']}-Hkv{s['Hkv']}-ds{s['d_store']}-dsel{s['d_sel']}-k{s['k']}"
            f"-T{s['T']}-ch{'+'.join(str(x) for x in s['chunks'])}-cap{s['T_cap']}")


@pytest.mark.parametrize("s", PREFILL_SHAPES, ids=[_pid(s) for s in PREFILL_SHAPES])
def test_shape_sweep_prefill(s):
    B, Hq, Hkv, T, k = s["B"], s["Hq"], s["Hkv"], s["T"], s["k"]
    d_store, d_sel = s["d_store"], s["d_sel"]
    c = config(4, B=B, Hq=Hq, Hkv=Hkv, T=T, k=k, d_store=d_store, d_sel=d_sel)
    d = c["d"]
    inp = make_prefill_inputs(c)
    kp, v = new_cache(B, Hkv, d, d_store, s["T_cap"], "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    out = torch.full((B, Hq, T, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, T, d), float("nan"), device=DEV)
    mask = torch.zeros(B, Hq, T, d // 32, dtype=torch.int32, device=DEV)
    c0 = 0
    for L in s["chunks"]:
        aq.aqua_project_keys(cache, inp["k"][:, :, c0:c0 + L].contiguous().to(DEV),
                             inp["v"][:, :, c0:c0 + L].contiguous().to(DEV), P, L)
        ws = torch.empty(aq.aqua_prefill_workspace(cache, Hq, L), dtype=torch.uint8, device=DEV)
        o = torch.empty(B, Hq, L, d, device=DEV)
        qpc = torch.empty(B, Hq, L, d, device=DEV)
        mc = torch.empty(B, Hq, L, d // 32, dtype=torch.int32, device=DEV)
        aq.aqua_prefill_chunk(cache, Hq, inp["q"][:, :, c0:c0 + L].contiguous().to(DEV), L, c0, P,
                              d_sel, k, 1 / math.sqrt(d), o, ws=ws, q_proj_out=qpc, mask_out=mc)
        out[:, :, c0:c0 + L] = o
        qp[:, :, c0:c0 + L] = qpc
        mask[:, :, c0:c0 + L] = mc
        c0 += L
    torch.cuda.synchronize()
    assert cache.len == T

    m = unpack_mask(mask, d)
    assert np.array_equal(m, O.select(qp.cpu().double().numpy(), d_sel, k))
    P64 = storage_to_f64(inp["P"])
    G = Hq // Hkv
    got = out.cpu().double().numpy()
    for b in range(B):
        for g in range(Hkv):
            Kp = O.project_keys_stored(storage_to_f64(inp["k"][b, g]), P64, "bf16", d_store)
            V = storage_to_f64(inp["v"][b, g])
            for h in range(g * G, (g + 1) * G):
                qph = O.project(storage_to_f64(inp["q"][b, h]), P64)
                ref = np.stack([O.attend(qph[p], m[b, h, p], Kp[:p + 1], V[:p + 1],
                                         1 / math.sqrt(d))[0] for p in range(T)])
                assert_close(got[b, h], ref, "bf16", f"prefill b{b} h{h}")
