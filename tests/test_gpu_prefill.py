"""GPU parity of aqua_prefill_chunk (per-query selection + causal MFMA attention) against the
oracle: masks bit-exact given the GPU's q', outputs within the bf16 tolerance."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import DEV, assert_close, new_cache, unpack_mask
from oracle import aqua_oracle as O
from synth import config, make_prefill_inputs, storage_to_f64

pytestmark = pytest.mark.gpu


def _run_chunks(inp, c, chunk, T_cap=None, d_store=None, d_sel=None, k=None):
    """Append each chunk's keys, then prefill its queries.  Returns GPU out, q', masks.
    chunk: a chunk length, or the list of chunk lengths."""
    B, Hq, Hkv, d, T = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"]
    d_store = d_store or d
    d_sel = d_sel or d_store
    k = k or c["k"]
    T_cap = T_cap or ((T + 63) // 64 * 64)
    kp, v = new_cache(B, Hkv, d, d_store, T_cap, "bf16")
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    out = torch.full((B, Hq, T, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, T, d), float("nan"), device=DEV)
    mask = torch.zeros(B, Hq, T, d // 32, dtype=torch.int32, device=DEV)
    lengths = chunk if isinstance(chunk, (list, tuple)) else \
        [min(chunk, T - c0) for c0 in range(0, T, chunk)]
    assert sum(lengths) == T
    c0 = 0
    for L in lengths:
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
    return out, qp, mask


def _oracle_rows(inp, c, m, rows, d_store=None):
    """Oracle output for (b, h, position) rows, with the given masks."""
    d = c["d"]
    d_store = d_store or d
    G = c["Hq"] // c["Hkv"]
    P64 = storage_to_f64(inp["P"])
    cacheK = {}
    res = []
    for b, h, p in rows:
        g = h // G
        if (b, g) not in cacheK:
            cacheK[(b, g)] = (O.project_keys_stored(storage_to_f64(inp["k"][b, g]), P64, "bf16",
                                                    d_store),
                              storage_to_f64(inp["v"][b, g]))
        Kp, V = cacheK[(b, g)]
        qp = O.project(storage_to_f64(inp["q"][b, h, p]), P64)
        o, _ = O.attend(qp, m[b, h, p], Kp[:p + 1], V[:p + 1], 1 / math.sqrt(d))
        res.append(o)
    return np.stack(res)


def _check(inp, c, out, qp, mask, rows, d_sel, k, d_store=None):
    d = c["d"]
    m = unpack_mask(mask, d)
    assert np.array_equal(m, O.select(qp.cpu().double().numpy(), d_sel, k))
    ref = _oracle_rows(inp, c, m, rows, d_store)
    got = np.stack([out[b, h, p].cpu().double().numpy() for b, h, p in rows])
    assert_close(got, ref, "bf16", "prefill rows")


@pytest.mark.parametrize("Hq,Hkv,T,chunk,k", [
    (8, 2, 300, 300, 96),     # one ragged chunk
    (8, 2, 700, 256, 96),     # chunks, ragged tail
    (4, 4, 333, 128, 64),     # G = 1
    (8, 4, 260, 100, 128),    # G = 2, k = d
    (16, 2, 200, 200, 32),    # G = 8
    # chunks that are multiples of 64 at G >= 4 take the paired form (blocks j and last - j)
    (8, 2, 1024, 512, 96),    # two chunks of 16 blocks
    (16, 2, 640, 128, 64),    # G = 8, five chunks of 4 blocks
    (8, 2, 512, [32, 128, 256, 96], 96),  # paired chunks starting at 32 and 160
    (1, 1, 77, 77, 96),       # 154 query rows: the last 32-row selection block holds 26, so one
                              # wavefront of the selection has 2 rows and one has none
])
def test_prefill_small_all_rows(Hq, Hkv, T, chunk, k):
    c = config(4, B=2, Hq=Hq, Hkv=Hkv, T=T, k=k)
    inp = make_prefill_inputs(c)
    out, qp, mask = _run_chunks(inp, c, chunk)
    rows = [(b, h, p) for b in range(c["B"]) for h in range(Hq) for p in range(T)]
    _check(inp, c, out, qp, mask, rows, c["d"], k)


def _plateau_inputs(c, mu=6.0, l0=33.0, l1=16.0):
    """Inputs whose scores climb in two jumps: every query gets a common component mu*u (u a
    seeded unit vector), keys 0..63 are -l0*u and keys 64..511 are -l1*u (identical keys, so
    equal scores), the rest are the generator's.  A row's running max starts near -22 (log2
    units) from tile 0, jumps to near -11 at position 64 and to the generator's scale (~2) at
    position 512: two moves past the kernel's 8-unit slack, one of them inside the causally
    masked steps of the workgroups that hold position 512."""
    inp = make_prefill_inputs(c)
    u = np.random.default_rng(2024).standard_normal(c["d"])
    u = torch.from_numpy(u / np.linalg.norm(u))
    dt = inp["q"].dtype
    inp["q"] = (inp["q"].double() + mu * u).to(dt)
    k = inp["k"].double()
    k[:, :, :64] = -l0 * u
    k[:, :, 64:512] = -l1 * u
    inp["k"] = k.to(dt)
    return inp


@pytest.mark.parametrize("chunk", [512, 300, [448, 128, 448]])
def test_prefill_running_max_moves(chunk):
    """The online softmax's running max moving past its slack, in unmasked steps (the next
    tile's scores checked before use) and in masked ones (the tile's own scores, with the
    already computed next tile shifted too).  512-token chunks take the paired form, 300 the
    consecutive one; [448, 128, 448] puts position 512 at a chunk's masked diagonal."""
    c = config(4, B=1, Hq=8, Hkv=2, T=1024, k=96)
    inp = _plateau_inputs(c)
    # the jumps are there: scores of row 900 (oracle arithmetic) at keys 5, 100 and 700
    P64 = storage_to_f64(inp["P"])
    Kp = O.project_keys_stored(storage_to_f64(inp["k"][0, 0]), P64, "bf16", c["d"])
    qp = O.project(storage_to_f64(inp["q"][0, 0, 900]), P64)
    sel = O.select(qp[None], c["d"], 96)[0]
    s = (np.where(sel, qp, 0) @ Kp.T) / math.sqrt(c["d"]) / math.log(2)
    assert s[100] - s[5] > 8 and s[:901].max() - s[100] > 8
    out, qp_g, mask = _run_chunks(inp, c, chunk)
    rows = [(0, h, p) for h in range(8) for p in range(c["T"])]
    _check(inp, c, out, qp_g, mask, rows, c["d"], 96)


def test_prefill_memory_cut():
    """AQUA-Memory: K' keeps dims 0..95, top-64 of those 96."""
    c = config(4, B=1, Hq=8, Hkv=2, T=400, k=64)
    inp = make_prefill_inputs(c)
    out, qp, mask = _run_chunks(inp, c, 160, d_store=96, d_sel=96, k=64)
    rows = [(0, h, p) for h in range(8) for p in range(400)]
    _check(inp, c, out, qp, mask, rows, 96, 64, d_store=96)


def test_prefill_q_proj_fp32_accuracy():
    """The prefill's q' (bf16 MFMA with P split into three bf16 parts) is within the fp32
    summation bound of the fp64 product of the same inputs: |dq'_i| <= gamma_n sum_j |q_j P_ji|
    with n = 3 d + 1 accumulations (gamma_n = n u / (1 - n u), u = 2^-24); its masks are the
    oracle's selection of it (checked in _check)."""
    c = config(4, B=1, Hq=8, Hkv=2, T=500, k=96)
    inp = make_prefill_inputs(c)
    out, qp, mask = _run_chunks(inp, c, 500)
    q64 = storage_to_f64(inp["q"]).reshape(-1, 128)
    P64 = storage_to_f64(inp["P"])
    ref = q64 @ P64
    n = 3 * 128 + 1
    gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    bound = gamma * (np.abs(q64) @ np.abs(P64))
    err = np.abs(qp.reshape(-1, 128).cpu().double().numpy() - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    rows = [(0, h, p) for h in range(8) for p in range(0, 500, 7)]
    _check(inp, c, out, qp, mask, rows, 128, 96)


def test_prefill_llama8b_t16384():
    """The chunked-prefill workload (T=16384 in 8 chunks of 2048, k=96): all 524288 masks
    bit-exact against the oracle's selection of the GPU's q'; 384 rows per chunk against the
    oracle, covering every head of every chunk (the first and last position of each chunk, and
    random ones); every output finite."""
    c = config(4)
    inp = make_prefill_inputs(c, workers=16)
    out, qp, mask = _run_chunks(inp, c, c["chunk"])
    T, Hq, chunk = c["T"], c["Hq"], c["chunk"]
    m = unpack_mask(mask, 128)
    assert np.array_equal(m.reshape(-1, 128),
                          O.select(qp.cpu().double().numpy().reshape(-1, 128), 128, 96))
    rng = np.random.default_rng(0)
    rows = []
    for c0 in range(0, T, chunk):
        for h in range(Hq):
            rows += [(0, h, c0), (0, h, c0 + chunk - 1)]
            rows += [(0, h, int(p)) for p in c0 + rng.integers(0, chunk, 10)]
    ref = _oracle_rows(inp, c, m, rows)
    out_np = out.cpu().numpy()
    got = np.stack([out_np[b, h, p].astype(np.float64) for b, h, p in rows])
    assert_close(got, ref, "bf16", "prefill T16384")
    assert torch.isfinite(out).all()


def test_prefill_q_proj_equals_select():
    """The prefill's q' and masks are aqua_select_dims' for the same bf16 rows, bit for bit (both
    run the library's one bf16 projection and the same selection)."""
    c = config(4, B=1, Hq=8, Hkv=2, T=640, k=96)
    inp = make_prefill_inputs(c)
    out, qp, mask = _run_chunks(inp, c, 320)
    q = inp["q"].reshape(-1, 128).to(DEV)
    qp2 = torch.empty(q.shape[0], 128, device=DEV)
    mask2 = torch.empty(q.shape[0], 4, dtype=torch.int32, device=DEV)
    aq.aqua_select_dims(q, inp["P"].to(DEV), 128, 96, qp2, mask2)
    torch.cuda.synchronize()
    assert torch.equal(qp.reshape(-1, 128), qp2)
    assert torch.equal(mask.reshape(-1, 4), mask2)


@pytest.mark.parametrize("d_sel,k", [(128, 96), (128, 5), (96, 40), (128, 127), (128, 128)])
def test_prefill_selection_ties(d_sel, k):
    """Many exact ties in |q'| (P = I, so q' = q: magnitudes from a tiny set, both signs, +-0;
    bf16 has no fp32 denormals to offer beyond its own): the prefill masks must be the oracle's
    selection of the GPU's q' (ties to the lower index), and the outputs still match."""
    c = config(4, B=1, Hq=8, Hkv=2, T=300, k=k)
    inp = make_prefill_inputs(c)
    rng = np.random.default_rng(11)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 0.25, -0.25, 2.0], dtype=np.float32)
    inp["q"] = torch.from_numpy(rng.choice(vals, size=tuple(inp["q"].shape))).to(torch.bfloat16)
    inp["P"] = torch.eye(128)
    out, qp, mask = _run_chunks(inp, c, 128, d_store=d_sel, d_sel=d_sel, k=k)
    rows = [(0, h, p) for h in range(8) for p in range(0, 300, 13)]
    _check(inp, c, out, qp, mask, rows, d_sel, k, d_store=d_sel)
