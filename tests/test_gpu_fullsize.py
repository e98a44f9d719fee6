"""The benchmarked decode kernels at the benchmarked shape, every head against the oracle: one
Llama-3.1-8B-shaped layer, B=16, Hq=32, Hkv=8, d_head=128, T=8192 bf16 tokens, k=96, in a cache of
capacity T + 256 = 8448 tokens (the capacity the benchmark allocates).  At this shape the
split-T kernel runs its 8-wavefront layout (128 groups x 2 full 4096-token splits: one
512-thread workgroup per CU of a 256-CU device), in both the plain (aqua_decode) and the fused
(aqua_decode_step) form.

Also here, on the same inputs: the workspace contract (no clearing, whatever it holds, across
shapes) and a repetition test of the cross-workgroup merge (every workgroup of a group publishes
its partials for the group's last one, on any XCD: repeated launches must give the same bits)."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import DEV, assert_close, new_cache, oracle_decode, unpack_mask
from oracle import aqua_oracle as O
from synth import config, make_decode_inputs, storage_to_f64

pytestmark = pytest.mark.gpu

T_CAP = 8192 + 256


@pytest.fixture(scope="module")
def full():
    c = config(2)
    inp = make_decode_inputs(c, workers=16)
    dev = {"P": inp["P"].to(DEV), "k": inp["k"].to(DEV), "v": inp["v"].to(DEV),
           "q": inp["q"].to(DEV)}
    return c, inp, dev


def _check_masks(mask, qp, d, k):
    m = unpack_mask(mask, d)
    assert np.array_equal(m, O.select(qp.cpu().double().numpy(), d, k))
    return m


def _cache_with(c, dev, n):
    """A fresh (NaN-poisoned) cache of capacity T_CAP holding the first n tokens."""
    kp, v = new_cache(c["B"], c["Hkv"], c["d"], c["d"], T_CAP, "bf16")
    cache = aq.make_cache(kp, v, 0)
    aq.aqua_project_keys(cache, dev["k"][:, :, :n].contiguous(), dev["v"][:, :, :n].contiguous(),
                         dev["P"], n)
    return cache, kp, v


def _select(c, dev):
    B, Hq, d, k = c["B"], c["Hq"], c["d"], c["k"]
    qp = torch.full((B * Hq, d), float("nan"), device=DEV)
    mask = torch.full((B * Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_select_dims(dev["q"].reshape(B * Hq, d), dev["P"], d, k, qp, mask)
    return qp, mask


def test_decode_step_fullsize_all_heads(full):
    """aqua_decode_step (the benchmark's one launch): the cache holds 8191 tokens, the step
    appends token 8191 and attends all 8192.  Every mask bit-exact against the oracle's selection
    of the GPU's q'; all 512 heads' outputs against the oracle; the new token's K' and V."""
    c, inp, dev = full
    B, Hq, Hkv, d, T, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"], c["k"]
    cache, kp, v = _cache_with(c, dev, T - 1)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_decode_step(cache, Hq, dev["q"], dev["k"][:, :, T - 1].contiguous(),
                        dev["v"][:, :, T - 1].contiguous(), dev["P"], d, k, 1 / math.sqrt(d),
                        out, ws, q_proj_out=qp, mask_out=mask)
    torch.cuda.synchronize()
    assert cache.len == T
    m = _check_masks(mask, qp, d, k)
    ref = oracle_decode(inp, c, m)
    assert_close(out.cpu().double().numpy(), ref, "bf16", "decode step, all heads")
    # the new token in the cache: K' within one bf16 ulp plus the fp32 summation bound, V exact
    P64 = storage_to_f64(inp["P"])
    kraw = storage_to_f64(inp["k"][:, :, T - 1])
    kn = O.project_keys_stored(kraw, P64, "bf16", d)
    got = storage_to_f64(kp[:, :, :, T - 1])
    bound = np.abs(kn) * 2.0 ** -7 + (3 * d + 1) * 2.0 ** -24 * (np.abs(kraw) @ np.abs(P64))
    assert np.all(np.abs(got - kn) <= bound)
    assert torch.equal(v[:, :, T - 1], dev["v"][:, :, T - 1])


def test_decode_fullsize_all_heads(full):
    """aqua_decode on aqua_select_dims' masks over all 8192 tokens: every mask and all 512
    heads against the oracle."""
    c, inp, dev = full
    B, Hq, d, T, k = c["B"], c["Hq"], c["d"], c["T"], c["k"]
    cache, _, _ = _cache_with(c, dev, T)
    qp, mask = _select(c, dev)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp, mask, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    m = _check_masks(mask.view(B, Hq, d // 32), qp.view(B, Hq, d), d, k)
    ref = oracle_decode(inp, c, m)
    assert_close(out.cpu().double().numpy(), ref, "bf16", "decode, all heads")


def test_workspace_needs_no_clearing(full):
    """One workspace, filled with random bytes and never cleared, serves calls of different
    lengths (the 8-wavefront layout at 8192 tokens, the 4-wavefront one at 6000 and at 3000) in
    turn: every call gives the bits of the same call on a zeroed workspace of its own,
    and those are checked against the oracle on a sample of heads."""
    c, inp, dev = full
    B, Hq, d, k = c["B"], c["Hq"], c["d"], c["k"]
    cache, _, _ = _cache_with(c, dev, c["T"])
    qp, mask = _select(c, dev)
    n = aq.aqua_decode_workspace(cache, Hq)
    g = torch.Generator(device="cpu").manual_seed(7)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    scale = 1 / math.sqrt(d)
    refs = {}
    for length in (8192, 6000, 3000):
        cache.len = length
        ws0 = torch.zeros(n, dtype=torch.uint8, device=DEV)
        o = torch.full((B, Hq, d), float("nan"), device=DEV)
        aq.aqua_decode(cache, Hq, qp, mask, scale, o, ws0)
        refs[length] = o
    torch.cuda.synchronize()
    m = unpack_mask(mask.view(B, Hq, d // 32), d)
    heads = [(0, 0), (3, 17), (9, 30), (15, 31)]
    for length, o in refs.items():
        ref = oracle_decode(inp, c, m, length=length, heads=heads)
        for b, h in heads:
            assert_close(o[b, h].cpu().double().numpy(), ref[b, h], "bf16", f"len {length}")
    for it, length in enumerate((8192, 6000, 3000, 6000, 8192, 3000, 8192)):
        cache.len = length
        o = torch.full((B, Hq, d), float("nan"), device=DEV)
        aq.aqua_decode(cache, Hq, qp, mask, scale, o, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, refs[length]), f"call {it} (len {length}) on the uncleared workspace"


def test_merge_repeatable(full):
    """The split merge hands partials between workgroups on different XCDs through relaxed
    system-scope stores and loads ordered by the arrival counter.  25 launches at each of two
    layouts (2 splits of 4096 tokens; 3 of 2048 with a ragged last one) on one workspace must all
    give the first launch's bits; the run stops at the first that does not."""
    c, inp, dev = full
    B, Hq, d = c["B"], c["Hq"], c["d"]
    cache, _, _ = _cache_with(c, dev, c["T"])
    qp, mask = _select(c, dev)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    scale = 1 / math.sqrt(d)
    for length in (8192, 5000):
        cache.len = length
        first = torch.empty(B, Hq, d, device=DEV)
        aq.aqua_decode(cache, Hq, qp, mask, scale, first, ws)
        for it in range(25):
            o = torch.full_like(first, float("nan"))
            aq.aqua_decode(cache, Hq, qp, mask, scale, o, ws)
            torch.cuda.synchronize()
            assert torch.equal(o, first), f"launch {it} at len {length} differs"


@pytest.mark.skip(reason="a GPU run that included this test ended with a GPU memory fault (with "
                         "an epoch-tagged partial hand-off since removed from the kernels); the "
                         "box ended before its log came back and no cause was shown, so graph "
                         "replay of the decode kernel stays off the GPU")
def test_decode_graph_replay(full):
    """aqua_decode captured in a HIP graph: every replay runs with the epoch taken at capture, so
    the partial words the previous replay left carry this replay's tag; each replay must still
    give the bits of an eager call on the same inputs (the group's last workgroup zeroes the words
    it consumed).  The queries change in place between replays (q' scaled: same masks, other
    weights), so a stale partial would show, and an eager call on the same workspace runs between
    replays (other epochs in the words and counters)."""
    c, inp, dev = full
    B, Hq, d = c["B"], c["Hq"], c["d"]
    cache, _, _ = _cache_with(c, dev, c["T"])
    qp, mask = _select(c, dev)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    scale = 1 / math.sqrt(d)
    qbuf = qp.clone()
    out = torch.empty(B, Hq, d, device=DEV)
    aq.aqua_decode(cache, Hq, qbuf, mask, scale, out, ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aq.aqua_decode(cache, Hq, qbuf, mask, scale, out, ws)
    torch.cuda.synchronize()
    for it, f in enumerate((1.0, 0.5, 2.0, 1.0, 3.0, 0.25, 1.5)):
        qbuf.copy_(qp * f)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.full_like(out, float("nan"))
        aq.aqua_decode(cache, Hq, qbuf, mask, scale, ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {it} (q' x {f}) differs from the eager call"


@pytest.mark.parametrize("n", [2048, 4096])
def test_short_lengths_large_batch(full, n):
    """At B16 and up to 4096 tokens the short kernel's grid (256-token workgroups) would fill more
    than two rounds of the device, so both forms run the split-T kernel there: the fused step over
    n tokens (a cache of n - 1 plus the new one) and then the decode over the same n, every mask
    bit-exact, sampled heads against the oracle."""
    c, inp, dev = full
    B, Hq, d, k = c["B"], c["Hq"], c["d"], c["k"]
    cache, kp, v = _cache_with(c, dev, n - 1)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    scale = 1 / math.sqrt(d)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_decode_step(cache, Hq, dev["q"], dev["k"][:, :, n - 1].contiguous(),
                        dev["v"][:, :, n - 1].contiguous(), dev["P"], d, k, scale, out, ws,
                        q_proj_out=qp, mask_out=mask)
    torch.cuda.synchronize()
    assert cache.len == n
    m = _check_masks(mask, qp, d, k)
    heads = [(0, 0), (3, 17), (7, 5), (9, 30), (15, 31)]
    ref = oracle_decode(inp, c, m, length=n, heads=heads)
    out2 = torch.full_like(out, float("nan"))
    aq.aqua_decode(cache, Hq, qp.view(B * Hq, d), mask.view(B * Hq, d // 32), scale, out2, ws)
    torch.cuda.synchronize()
    for b, h in heads:
        assert_close(out[b, h].cpu().double().numpy(), ref[b, h], "bf16", f"step, len {n}")
        assert_close(out2[b, h].cpu().double().numpy(), ref[b, h], "bf16", f"decode, len {n}")
    assert torch.isfinite(out).all() and torch.isfinite(out2).all()


@pytest.mark.parametrize("T", [4097, 8193, 16384])
def test_step_b16_layouts(T):
    """The fused step at batch 16 (128 groups) where the layout rule picks other grids than the
    benchmark's: 4097 tokens (no full 8-wavefront split per group: the 4-wavefront layout, 3
    splits of 2048), 8193 (the 8-wavefront grid would end on a half round: 4-wavefront, 5 splits)
    and 16384 (8-wavefront, 4 splits of 4096 filling two whole rounds).  At 8193 the grid (640
    workgroups) takes more than one round of resident workgroups, so every group's one-token last
    split is dealt after all the full ones.  Every mask against the oracle's selection of the
    GPU's q'; the output of the step, and of aqua_decode over the same tokens, on a sample of heads
    in every group."""
    c = config(2, T=T)
    inp = make_decode_inputs(c, workers=16)
    B, Hq, Hkv, d, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["k"]
    T_cap = T + 256 - T % 64
    kp, v = new_cache(B, Hkv, d, d, T_cap, "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                         inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_decode_step(cache, Hq, inp["q"].to(DEV), inp["k"][:, :, T - 1].contiguous().to(DEV),
                        inp["v"][:, :, T - 1].contiguous().to(DEV), P, d, k, 1 / math.sqrt(d),
                        out, ws, q_proj_out=qp, mask_out=mask)
    torch.cuda.synchronize()
    assert cache.len == T
    m = _check_masks(mask.view(B * Hq, d // 32), qp.view(B * Hq, d), d, k).reshape(B, Hq, d)
    heads = [(b, 4 * g + (b + g) % 4) for b in range(B) for g in range(Hkv)]  # one per group
    ref = oracle_decode(inp, c, m, heads=heads)
    # aqua_decode over the same T tokens with the step's q' and masks: the plain kernel's grid
    out2 = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp, mask, 1 / math.sqrt(d), out2, ws)
    torch.cuda.synchronize()
    for name, o in (("aqua_decode_step", out), ("aqua_decode", out2)):
        got = o.cpu().double().numpy()
        for b, h in heads:
            assert_close(got[b, h], ref[b, h], "bf16", f"{name}, T {T}, batch {b}, head {h}")


def test_step_one_kv_head_shard():
    """The benchmark layer's share on one GPU of eight when KV heads are sharded (B16, Hq4,
    Hkv1, T8192): 16 groups of 4 splits of 2048 tokens, 64 four-wavefront workgroups.  Every mask
    and every head against the oracle; aqua_decode over the same tokens too."""
    c = config(2, Hq=4, Hkv=1, T=8192)
    inp = make_decode_inputs(c, workers=16)
    B, Hq, Hkv, d, k, T = c["B"], c["Hq"], c["Hkv"], c["d"], c["k"], c["T"]
    kp, v = new_cache(B, Hkv, d, d, T_CAP, "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                         inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_decode_step(cache, Hq, inp["q"].to(DEV), inp["k"][:, :, T - 1].contiguous().to(DEV),
                        inp["v"][:, :, T - 1].contiguous().to(DEV), P, d, k, 1 / math.sqrt(d),
                        out, ws, q_proj_out=qp, mask_out=mask)
    out2 = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp, mask, 1 / math.sqrt(d), out2, ws)
    torch.cuda.synchronize()
    m = _check_masks(mask.view(B * Hq, d // 32), qp.view(B * Hq, d), d, k).reshape(B, Hq, d)
    ref = oracle_decode(inp, c, m)
    assert_close(out.cpu().double().numpy(), ref, "bf16", "shard step, all heads")
    assert_close(out2.cpu().double().numpy(), ref, "bf16", "shard decode, all heads")


def test_step_tail_last_two_level():
    """Batch 4 at 40000 tokens: 32 groups of 20 splits of 2048 (640 four-wavefront workgroups, the
    last split of each group partial), so the grid takes more than one round and the groups' last
    splits are dealt after all the full ones, with the merge in two levels (runs of 8 splits).
    Every mask, and two heads of every group for the fused step and aqua_decode, against the
    oracle."""
    c = config(2, B=4, T=40000)
    inp = make_decode_inputs(c, workers=16)
    B, Hq, Hkv, d, k, T = c["B"], c["Hq"], c["Hkv"], c["d"], c["k"], c["T"]
    T_cap = T + 256 - T % 64
    kp, v = new_cache(B, Hkv, d, d, T_cap, "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                         inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    aq.aqua_decode_step(cache, Hq, inp["q"].to(DEV), inp["k"][:, :, T - 1].contiguous().to(DEV),
                        inp["v"][:, :, T - 1].contiguous().to(DEV), P, d, k, 1 / math.sqrt(d),
                        out, ws, q_proj_out=qp, mask_out=mask)
    out2 = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp, mask, 1 / math.sqrt(d), out2, ws)
    torch.cuda.synchronize()
    m = _check_masks(mask.view(B * Hq, d // 32), qp.view(B * Hq, d), d, k).reshape(B, Hq, d)
    heads = [(b, 4 * g + j) for b in range(B) for g in range(Hkv) for j in ((b + g) % 4, 3 - (b + g) % 4)]
    ref = oracle_decode(inp, c, m, heads=heads)
    for name, o in (("aqua_decode_step", out), ("aqua_decode", out2)):
        got = o.cpu().double().numpy()
        for b, h in heads:
            assert_close(got[b, h], ref[b, h], "bf16", f"{name}, batch {b}, head {h}")
