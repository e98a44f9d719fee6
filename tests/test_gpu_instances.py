"""Every compiled form of the decode kernels against the oracle.

The library builds one kernel per (storage dtype, d, group size G) for each decode form: the
short-context kernel, the fused short step, the split-T kernel (plain and fused, in each of its
workgroup layouts) and the H2O step.  The matrix below drives each of them: for every dtype,
d and G, the fused step appends token T-1 to a cache of T-1 tokens and decodes, then aqua_decode
runs on the same cache with the step's q' and masks, once at 1500 tokens (short-context kernels)
and once at 5000 (split-T, 4 wavefronts per workgroup).  Larger shapes take the 8-wavefront
split-T layout in the forms the benchmark does not: G = 4 with fp32 storage at d = 128 and
d = 64 and with bf16 at d = 64, and G = 8 in all four.  Each output is checked against the
oracle (all heads in the matrix, sampled heads of every group in the large shapes), the masks
against the oracle's selection of the GPU's q', and the appended token's K' and V; a one-token
aqua_project_keys of the same token is checked the same way.  The streaming-read probe's result (the XOR of every
32-bit word of each workgroup's slice) is checked against the host's."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import DEV, assert_close, new_cache, oracle_decode, unpack_mask
from oracle import aqua_oracle as O
from synth import config, make_decode_inputs, storage_to_f64

pytestmark = pytest.mark.gpu


def _check_appended(inp, kp_col, v_col, k_in, v_in, d, d_store, dtype):
    """kp_col [B][Hkv][d_store] and v_col [B][Hkv][d] (GPU) against the oracle's projection of
    the raw key k_in [B][Hkv][d] (one storage rounding plus the fp32 sum's bound) and v_in."""
    P64 = storage_to_f64(inp["P"])
    kin = storage_to_f64(k_in)
    kn = O.project_keys_stored(kin, P64, dtype, d_store)
    got = storage_to_f64(kp_col)
    ulp = np.abs(kn) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)
    acc = (d * 2.0 ** -24 * (np.abs(kin) @ np.abs(P64)))[..., :d_store]
    assert np.all(np.abs(got - kn) <= ulp + acc)
    assert np.array_equal(storage_to_f64(v_col), storage_to_f64(v_in))


def _step_then_decode(c, heads=None):
    B, Hq, Hkv, d, T, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"], c["k"]
    dtype = c["dtype"]
    inp = make_decode_inputs(c)
    kp, v = new_cache(B, Hkv, d, d, (T + 63) // 64 * 64, dtype)
    cache = aq.make_cache(kp, v, 0)
    P = inp["P"].to(DEV)
    aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                         inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
    ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    qp = torch.full((B, Hq, d), float("nan"), device=DEV)
    mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    k_new = inp["k"][:, :, T - 1].contiguous()
    v_new = inp["v"][:, :, T - 1].contiguous()
    aq.aqua_decode_step(cache, Hq, inp["q"].to(DEV), k_new.to(DEV), v_new.to(DEV), P, d, k,
                        scale, out, ws, q_proj_out=qp, mask_out=mask)
    out2 = torch.full((B, Hq, d), float("nan"), device=DEV)
    aq.aqua_decode(cache, Hq, qp.reshape(B * Hq, d), mask.reshape(B * Hq, d // 32), scale, out2,
                   ws)
    # the same token alone through aqua_project_keys (the few-token kernel)
    kp1, v1 = new_cache(B, Hkv, d, d, 64, dtype)
    aq.aqua_project_keys(aq.make_cache(kp1, v1, 0), k_new[:, :, None].contiguous().to(DEV),
                         v_new[:, :, None].contiguous().to(DEV), P, 1)
    torch.cuda.synchronize()
    assert cache.len == T

    m = unpack_mask(mask, d)
    assert np.array_equal(m, O.select(qp.cpu().double().numpy(), d, k))
    ref = oracle_decode(inp, c, m, heads=heads)
    hl = heads or [(b, h) for b in range(B) for h in range(Hq)]
    o1, o2 = out.cpu().double().numpy(), out2.cpu().double().numpy()
    for b, h in hl:
        assert_close(o1[b, h], ref[b, h], dtype, f"step ({b}, {h})")
        assert_close(o2[b, h], ref[b, h], dtype, f"decode ({b}, {h})")
    _check_appended(inp, kp[:, :, :, T - 1], v[:, :, T - 1], k_new, v_new, d, d, dtype)
    _check_appended(inp, kp1[:, :, :, 0], v1[:, :, 0], k_new, v_new, d, d, dtype)


@pytest.mark.parametrize("T", [1500, 5000])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_instance_matrix(dtype, d, G, T):
    c = config(2 if d == 128 else 1, B=1, Hq=2 * G, Hkv=2, d=d, T=T, k=3 * d // 4, d_store=d,
               d_sel=d, dtype=dtype)
    _step_then_decode(c)


@pytest.mark.parametrize("dtype,d,B,T,G", [
    ("f32", 128, 4, 16384, 4),   # 32 groups x 8 splits of 2048 tokens: 256 workgroups
    ("f32", 64, 4, 16384, 4),
    ("bf16", 64, 4, 32768, 4),   # 32 groups x 8 splits of 4096 tokens
    ("bf16", 128, 4, 32768, 8),  # G = 8 takes the same layout
    ("bf16", 64, 4, 32768, 8),
    ("f32", 128, 4, 16384, 8),
    ("f32", 64, 4, 16384, 8),
])
def test_eight_wave_layout_forms(dtype, d, B, T, G):
    c = config(2 if d == 128 else 1, B=B, Hq=8 * G, Hkv=8, d=d, T=T, k=3 * d // 4, d_store=d,
               d_sel=d, dtype=dtype)
    heads = [(b, G * g + (b + g) % G) for b in range(B) for g in range(8)]
    _step_then_decode(c, heads=heads)


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 7), ((1 << 16) + 16 * 5, 3), (4096, 9),
                                           (64, 3)])  # the last slice empty
def test_stream_read_probe_result(nbytes, blocks):
    """Workgroup b reads 16-byte pieces [b p, (b + 1) p) of the buffer, p = ceil(pieces /
    blocks), and writes the XOR of their 32-bit words (0 for a slice past the end)."""
    g = torch.Generator().manual_seed(nbytes + blocks)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    sink = torch.full((blocks,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    aq.aqua_stream_read_probe(host.to(DEV), blocks, sink)
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32)
    n16 = nbytes // 16
    per = (n16 + blocks - 1) // blocks
    want = []
    for b in range(blocks):
        lo, hi = min(b * per, n16), min((b + 1) * per, n16)
        want.append(int(np.bitwise_xor.reduce(words[4 * lo:4 * hi])) if hi > lo else 0)
    assert sink.cpu().numpy().view(np.uint32).tolist() == want
