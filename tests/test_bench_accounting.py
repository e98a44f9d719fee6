"""bench.py's algorithmic byte counts (the numerator of roofline.achieved) against a brute-force
count over explicit masks, and its single-GPU contract.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _masks(rng, B, Hq, d, k):
    """Random per-head selections of k of d dims, as the library's mask words [B][Hq][d/32]."""
    sel = np.zeros((B, Hq, d), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            sel[b, h, rng.choice(d, k, replace=False)] = True
    words = np.zeros((B, Hq, d // 32), dtype=np.uint32)
    for i in range(d):
        words[:, :, i // 32] |= sel[:, :, i].astype(np.uint32) << np.uint32(i % 32)
    return sel, words.view(np.int32)


@pytest.mark.parametrize("B,Hq,Hkv,d,d_store,k", [(2, 8, 2, 128, 128, 96), (3, 4, 4, 64, 64, 40),
                                                  (1, 16, 2, 128, 96, 32)])
def test_union_rows_brute_force(B, Hq, Hkv, d, d_store, k):
    rng = np.random.default_rng(7)
    sel, words = _masks(rng, B, Hq, d, k)
    G = Hq // Hkv
    U = bench.union_rows(words, B, Hkv, G, d, d_store)
    for b in range(B):
        for g in range(Hkv):
            dims = set()
            for h in range(g * G, (g + 1) * G):
                dims |= {i for i in range(d_store) if sel[b, h, i]}
            assert U[b, g] == len(dims)


def test_decode_and_step_bytes_brute_force():
    """Every byte a decode launch must move, counted item by item: each (b, g) reads T tokens
    of each K' row in its union and all T V rows, reads q' (fp32) and masks, writes out (fp32).
    The fused step reads T - 1 cached tokens, the raw q, the new k and v, P, and writes the new
    K' column and V row."""
    rng = np.random.default_rng(3)
    c = {"B": 2, "Hq": 8, "Hkv": 2, "d": 128, "d_store": 128, "dtype": "bf16"}
    B, Hq, Hkv, d = c["B"], c["Hq"], c["Hkv"], c["d"]
    T, es = 1000, 2
    sel, words = _masks(rng, B, Hq, d, 96)
    U = bench.union_rows(words, B, Hkv, Hq // Hkv, d, d)
    n = 0
    for b in range(B):
        for g in range(Hkv):
            n += U[b, g] * T * es   # K' rows of the union
            n += T * d * es         # V rows
    n += B * Hq * d * 4             # q' in
    n += B * Hq * (d // 32) * 4     # masks in
    n += B * Hq * d * 4             # out
    assert bench.decode_bytes(U, c, T) == n
    m = 0
    for b in range(B):
        for g in range(Hkv):
            m += U[b, g] * (T - 1) * es + (T - 1) * d * es
            m += 2 * d * es              # new k, v in
            m += (d + d) * es            # new K' column, V row out (d_store = d)
    m += B * Hq * d * es                 # raw q in
    m += d * d * 4                       # P
    m += B * Hq * d * 4                  # out
    assert bench.step_bytes(U, c, T) == m


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
