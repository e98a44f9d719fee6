"""GPU parity of aqua_select_dims and aqua_project_keys against the oracle (through the C ABI)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import DEV, new_cache, select, unpack_mask
from oracle import aqua_oracle as O
from synth import gen, storage_to_f64, to_storage

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _queries(cid, N, d, tau, dtype, P64, seed=0):
    raw, _ = gen.make_qk_block(cid, "q", (seed, 99), N, d, tau, P64)
    return to_storage(raw, dtype)


@pytest.mark.parametrize("d,d_sel,k,dtype,N", [
    (64, 64, 48, "f32", 5),
    (128, 128, 96, "bf16", 1001),
    (128, 96, 64, "bf16", 517),
    (128, 128, 1, "f32", 130),
    (128, 128, 128, "bf16", 64),
    (128, 128, 32, "bf16", 999),
    (64, 40, 7, "bf16", 77),
])
def test_select_matches_oracle(d, d_sel, k, dtype, N):
    P64 = gen.make_projection(2, d)
    P32 = torch.from_numpy(P64.astype(np.float32))
    q = _queries(2, N, d, 40.0, dtype, P64)
    qp, mask, idx = select(q.to(DEV), P32.to(DEV), d_sel, k, want_idx=True)
    torch.cuda.synchronize()
    qp_g = qp.cpu().double().numpy()
    m_g = unpack_mask(mask, d)
    # bit-exact against the oracle fed the GPU's q'
    assert np.array_equal(m_g, O.select(qp_g, d_sel, k))
    assert (m_g.sum(1) == k).all() and not m_g[:, d_sel:].any()
    # q' itself: fp32 accumulation of the stored inputs' exact products (bf16: 3 d products of q
    # with P's three bf16 parts; fp32: d fmas), |dq'_i| <= gamma_(3d+1) sum_j |q_j P_ji|
    q64, P64s = storage_to_f64(q), storage_to_f64(P32)
    qp64 = O.project(q64, P64s)
    n = 3 * d + 1
    bound = n * 2.0 ** -24 / (1 - n * 2.0 ** -24) * (np.abs(q64) @ np.abs(P64s))
    assert np.all(np.abs(qp_g - qp64) <= bound)
    # idx: the kept dims in ascending order
    ix = idx.cpu().numpy().astype(np.int64)
    for r in range(N):
        assert np.array_equal(ix[r], np.nonzero(m_g[r])[0])


def test_select_golden_ties():
    """Hand-worked tie cases with P = I (q' = q exactly), zero-padded to d = 64."""
    with open(os.path.join(GOLDEN, "select_ties.json")) as f:
        cases = json.load(f)["cases"]
    P = torch.eye(64, device=DEV)
    for c in cases:
        q = torch.zeros(1, 64)
        q[0, :len(c["q"])] = torch.tensor(c["q"], dtype=torch.float64).float()
        _, mask, _ = select(q.to(DEV), P, c["d_sel"], c["k"])
        got = unpack_mask(mask, 64)[0]
        assert list(got[:len(c["mask"])]) == c["mask"] and not got[len(c["mask"]):].any(), c["why"]


def test_select_constructed_ties_large():
    """Many exact ties (magnitudes from a tiny set, both signs, +-0, denormals) with P = I."""
    rng = np.random.default_rng(3)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 2.0 ** -149, -(2.0 ** -149), 3.0],
                    dtype=np.float32)
    P = torch.eye(128, device=DEV)
    q = torch.from_numpy(rng.choice(vals, size=(300, 128)))
    for d_sel, k in [(128, 96), (128, 5), (100, 64), (128, 127)]:
        qp, mask, _ = select(q.to(DEV), P, d_sel, k)
        assert np.array_equal(unpack_mask(mask, 128), O.select(qp.cpu().double().numpy(), d_sel,
                                                               k))


def _ulp_bf16(x):
    _, e = np.frexp(x)
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


@pytest.mark.parametrize("dtype,d,d_store,n,len0,T_cap", [
    ("bf16", 128, 128, 300, 37, 512),
    ("bf16", 128, 96, 65, 0, 128),
    ("f32", 64, 64, 256, 0, 256),
    ("f32", 128, 128, 33, 100, 192),
    ("bf16", 64, 64, 1, 63, 64),
    ("bf16", 128, 128, 8, 5, 64),      # a few tokens at an unaligned column
    ("bf16", 128, 128, 16, 48, 64),    # largest few-token launch (one 16-row MFMA tile)
    ("bf16", 128, 96, 17, 0, 64),      # smallest tiled launch (bf16)
    ("bf16", 128, 128, 256, 0, 256),   # two whole 128-token tiles, aligned 16-byte writes
    ("bf16", 128, 128, 200, 8, 256),   # aligned start, ragged last tile
    ("bf16", 128, 128, 150, 0, 256),   # streamed: the tail's workgroup starts on an odd tile
    ("bf16", 64, 64, 200, 3, 256),     # d = 64 tiles (two wavefronts per column block)
    ("f32", 128, 96, 9, 0, 64),        # smallest tiled launch (fp32)
    ("f32", 128, 128, 1, 191, 192),    # a decode step filling the last column
])
def test_project_keys_append(dtype, d, d_store, n, len0, T_cap):
    B, Hkv = 2, 3
    P64 = gen.make_projection(4, d)
    P32 = torch.from_numpy(P64.astype(np.float32))
    rng = np.random.default_rng(5)
    K = to_storage(rng.standard_normal((B, Hkv, n, d)) * 2, dtype)
    V = to_storage(rng.standard_normal((B, Hkv, n, d)), dtype)
    kp, v = new_cache(B, Hkv, d, d_store, T_cap, dtype)
    cache = aq.make_cache(kp, v, len0)
    aq.aqua_project_keys(cache, K.to(DEV), V.to(DEV), P32.to(DEV), n)
    torch.cuda.synchronize()
    assert cache.len == len0 + n
    kp_h = storage_to_f64(kp)
    ref = O.project_keys_stored(storage_to_f64(K), storage_to_f64(P32), dtype, d_store)
    got = np.swapaxes(kp_h[:, :, :, len0:len0 + n], 2, 3)
    exact = O.project(storage_to_f64(K), storage_to_f64(P32))[..., :d_store]
    # |bf16(fp32 sum) - bf16(exact)| <= one ulp + the fp32 summation error bound
    # (3 d + 1) u sum|K||P| (bf16 keys: 3 d exact products with P's parts)
    acc_err = (3 * d + 1) * 2.0 ** -24 * (np.abs(storage_to_f64(K)) @
                                          np.abs(storage_to_f64(P32)))
    big = np.maximum(np.abs(exact), np.abs(got))
    ulp = _ulp_bf16(big) if dtype == "bf16" else big * 2.0 ** -23
    assert np.all(np.abs(got - ref) <= ulp + acc_err[..., :d_store]), \
        "K' further from the oracle than storage rounding plus fp32 summation allow"
    if dtype == "bf16":
        assert np.mean(got == ref) > 0.999
    assert np.array_equal(storage_to_f64(v)[:, :, len0:len0 + n], storage_to_f64(V))
    # columns outside [len0, len0 + n) untouched
    assert np.isnan(kp_h[:, :, :, :len0]).all() and np.isnan(kp_h[:, :, :, len0 + n:]).all()


@pytest.mark.parametrize("B,Hkv,d,d_store,n,len0,T_cap,groups", [
    (16, 8, 128, 128, 8191, 0, 8448, (0, 37, 64, 127)),  # the cache fill: runs of 64 and 63
    (16, 8, 128, 96, 4000, 8, 4096, (1, 90)),           # d_store cut: dims past it recomputed
    (16, 8, 64, 64, 3000, 64, 3072, (5, 66, 127)),       # d = 64: two wavefronts per column block
    (4, 8, 128, 128, 5000, 16, 5120, (0, 31)),           # runs of 12 and a last of 6
])
def test_project_keys_streamed_runs(B, Hkv, d, d_store, n, len0, T_cap, groups):
    """Bulk appends of whole tiles (bf16, no slots, aligned start) stream runs of tiles per
    workgroup; the ragged tail goes through the one-tile kernel.  Sampled (b, g) groups are
    checked in full against the oracle; V is copied exactly everywhere."""
    P64 = gen.make_projection(9, d)
    P32 = torch.from_numpy(P64.astype(np.float32))
    g = torch.Generator().manual_seed(11)
    K = (torch.randn(B, Hkv, n, d, generator=g) * 2).to(torch.bfloat16)
    V = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16)
    kp, v = new_cache(B, Hkv, d, d_store, T_cap, "bf16")
    cache = aq.make_cache(kp, v, len0)
    aq.aqua_project_keys(cache, K.to(DEV), V.to(DEV), P32.to(DEV), n)
    torch.cuda.synchronize()
    assert cache.len == len0 + n
    assert torch.equal(v[:, :, len0:len0 + n].cpu(), V)
    Pf = storage_to_f64(P32)
    for flat in groups:
        b, h = divmod(flat, Hkv)
        Kg = K[b, h].float().double().numpy()
        ref = O.project_keys_stored(Kg, Pf, "bf16", d_store)
        got = kp[b, h, :, len0:len0 + n].float().double().cpu().numpy().T
        exact = O.project(Kg, Pf)[..., :d_store]
        acc_err = (3 * d + 1) * 2.0 ** -24 * (np.abs(Kg) @ np.abs(Pf))[..., :d_store]
        big = np.maximum(np.abs(exact), np.abs(got))
        assert np.all(np.abs(got - ref) <= _ulp_bf16(big) + acc_err), (b, h)
        assert np.mean(got == ref) > 0.999, (b, h)
        kh = kp[b, h].float().cpu().numpy()
        assert np.isnan(kh[:, :len0]).all() and np.isnan(kh[:, len0 + n:]).all(), (b, h)


def test_project_keys_streamed_equals_few_token():
    """The streamed bulk append (runs of 8 and 7 tiles per workgroup here) and one-token appends
    give the same K' bits."""
    B, Hkv, d, n = 16, 8, 128, 1000
    P32 = torch.from_numpy(gen.make_projection(10, d).astype(np.float32)).to(DEV)
    g = torch.Generator().manual_seed(12)
    K = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16).to(DEV)
    V = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16).to(DEV)
    kp1, v1 = new_cache(B, Hkv, d, d, 1024, "bf16")
    kp2, v2 = new_cache(B, Hkv, d, d, 1024, "bf16")
    c1, c2 = aq.make_cache(kp1, v1, 0), aq.make_cache(kp2, v2, 0)
    aq.aqua_project_keys(c1, K, V, P32, n)
    for t in range(n):
        aq.aqua_project_keys(c2, K[:, :, t:t + 1].contiguous(), V[:, :, t:t + 1].contiguous(),
                             P32, 1)
    torch.cuda.synchronize()
    assert torch.equal(kp1[..., :n], kp2[..., :n])
    assert torch.equal(v1[:, :, :n], v2[:, :, :n])


@pytest.mark.parametrize("n", [5, 40])
def test_project_keys_slots(n):
    """Explicit destination columns (the H2O slot append): a few-token launch and a tiled one
    (the tiled kernel writes token by token where the columns are not consecutive)."""
    B, Hkv, d, T_cap = 1, 2, 128, 64
    P64 = gen.make_projection(6, d)
    P32 = torch.from_numpy(P64.astype(np.float32))
    rng = np.random.default_rng(6)
    K = to_storage(rng.standard_normal((B, Hkv, n, d)), "bf16")
    V = to_storage(rng.standard_normal((B, Hkv, n, d)), "bf16")
    perm = [np.random.default_rng(60 + g).permutation(T_cap)[:n] for g in range(Hkv)]
    slots = torch.from_numpy(np.stack(perm)[None].astype(np.int32))
    kp, v = new_cache(B, Hkv, d, d, T_cap, "bf16")
    cache = aq.make_cache(kp, v, 7)
    aq.aqua_project_keys(cache, K.to(DEV), V.to(DEV), P32.to(DEV), n, slots=slots.to(DEV))
    torch.cuda.synchronize()
    assert cache.len == 7
    ref = O.project_keys_stored(storage_to_f64(K), storage_to_f64(P32), "bf16", d)
    kp_h, v_h = storage_to_f64(kp), storage_to_f64(v)
    for g in range(Hkv):
        for t in range(n):
            col = int(slots[0, g, t])
            bound = _ulp_bf16(ref[0, g, t]) + (3 * d + 1) * 2.0 ** -24 * (
                np.abs(storage_to_f64(K)[0, g, t]) @ np.abs(storage_to_f64(P32)))
            assert np.all(np.abs(kp_h[0, g, :, col] - ref[0, g, t]) <= bound)
            assert np.array_equal(v_h[0, g, col], storage_to_f64(V)[0, g, t])
    written = np.zeros(T_cap, bool)
    written[slots[0, 0].numpy()] = True
    assert np.isnan(kp_h[0, 0, :, ~written]).all()


def test_project_keys_bulk_equals_few_token():
    """bf16 keys projected in one tiled launch and one at a time (the decode step's path) give the
    same K' bits: both run the library's one bf16 projection."""
    B, Hkv, d, n = 2, 2, 128, 40
    P32 = torch.from_numpy(gen.make_projection(8, d).astype(np.float32)).to(DEV)
    rng = np.random.default_rng(8)
    K = to_storage(rng.standard_normal((B, Hkv, n, d)), "bf16").to(DEV)
    kp1, v1 = new_cache(B, Hkv, d, d, 64, "bf16")
    kp2, v2 = new_cache(B, Hkv, d, d, 64, "bf16")
    c1, c2 = aq.make_cache(kp1, v1, 0), aq.make_cache(kp2, v2, 0)
    aq.aqua_project_keys(c1, K, None, P32, n)
    for t in range(n):
        aq.aqua_project_keys(c2, K[:, :, t:t + 1].contiguous(), None, P32, 1)
    torch.cuda.synchronize()
    assert torch.equal(kp1[..., :n], kp2[..., :n])
