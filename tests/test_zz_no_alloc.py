"""aqua_decode_step_noalloc (the decode step on the library's static scratch, for callers that
cannot allocate) against aqua_decode_step with a workspace of its own, through the C ABI: two
calls in a row, the second on a smaller input (so it finds the first one's contents in the
scratch), in plain and in mass mode.  Outputs, q', masks, the appended cache column and the
masses must be the same bits (the two run the same kernels); the outputs are also held to the
bf16 tolerance against the oracle on a sample of heads."""
import math

import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from gpu_util import DEV, assert_close, new_cache, oracle_decode, unpack_mask
from synth import config, make_decode_inputs

pytestmark = pytest.mark.gpu


def _step_both(c, T, T_cap, with_mass):
    """The same decode step (cache of T - 1 tokens, token T - 1 appended) through both entry
    points, each on its own copy of the cache."""
    inp = make_decode_inputs(c, workers=16)
    B, Hq, Hkv, d, k = c["B"], c["Hq"], c["Hkv"], c["d"], c["k"]
    d_store, d_sel = c["d_store"], c["d_sel"]
    P = inp["P"].to(DEV)
    q = inp["q"].to(DEV)
    kn = inp["k"][:, :, T - 1].contiguous().to(DEV)
    vn = inp["v"][:, :, T - 1].contiguous().to(DEV)
    runs = []
    mass0 = torch.rand(B, Hkv, T_cap, device=DEV) if with_mass else None
    for noalloc in (False, True):
        kp, v = new_cache(B, Hkv, d, d_store, T_cap, c["dtype"])
        cache = aq.make_cache(kp, v, 0)
        aq.aqua_project_keys(cache, inp["k"][:, :, :T - 1].contiguous().to(DEV),
                             inp["v"][:, :, :T - 1].contiguous().to(DEV), P, T - 1)
        out = torch.full((B, Hq, d), float("nan"), device=DEV)
        qp = torch.full((B, Hq, d), float("nan"), device=DEV)
        mask = torch.full((B, Hq, d // 32), -1, dtype=torch.int32, device=DEV)
        mass = mass0.clone() if with_mass else None
        if noalloc:
            aq.aqua_decode_step_noalloc(cache, Hq, q, kn, vn, P, d_sel, k, 1 / math.sqrt(d), out,
                                        mass=mass, q_proj_out=qp, mask_out=mask)
        else:
            ws = torch.empty(aq.aqua_decode_workspace(cache, Hq), dtype=torch.uint8, device=DEV)
            aq.aqua_decode_step(cache, Hq, q, kn, vn, P, d_sel, k, 1 / math.sqrt(d), out, ws,
                                mass=mass, q_proj_out=qp, mask_out=mask)
        torch.cuda.synchronize()
        assert cache.len == T
        runs.append(dict(out=out, qp=qp, mask=mask, kp=kp, v=v, mass=mass))
    ref, got = runs
    for r in runs:  # the cache columns past the step's are unwritten (NaN) in both
        r["kp"], r["v"] = r["kp"][..., :T], r["v"][:, :, :T]
    for name in ("out", "qp", "mask", "kp", "v") + (("mass",) if with_mass else ()):
        assert torch.equal(got[name], ref[name]), f"{name} differs from aqua_decode_step's"
    m = unpack_mask(got["mask"], d)
    heads = [(0, 0), (B - 1, Hq - 1), (B // 2, Hq // 3)]
    want = oracle_decode(inp, c, m, length=T, heads=heads)
    for b, h in heads:
        assert_close(got["out"][b, h].cpu().double().numpy(), want[b, h], c["dtype"],
                     f"noalloc head {(b, h)}")


@pytest.mark.parametrize("with_mass", [False, True])
def test_noalloc_two_calls_second_smaller(with_mass):
    # the benchmark's shape: split-T kernel, 8-wavefront layout (mass mode: 21.6 MB of scratch)
    c1 = config(2) if not with_mass else config(2, d_store=96, d_sel=96, k=64)
    _step_both(c1, 8192, 8192 + 256, with_mass)
    # then a smaller step (short-context kernel, 4 groups) on the scratch the first one left
    c2 = config(2, B=2, Hq=8, Hkv=2, T=3000)
    if with_mass:
        c2 = config(2, B=2, Hq=8, Hkv=2, T=3000, d_store=96, d_sel=96, k=64)
    _step_both(c2, 3000, 3008, with_mass)
