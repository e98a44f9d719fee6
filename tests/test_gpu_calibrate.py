"""GPU parity of the offline projection's Gram matrix (aqua_gram, through the C ABI) and of the
projection built from it (calibrate_projection) against the oracle's calibration.

Tolerances are the arithmetic's own bounds, not fitted: every product is exact (bf16 values, or
fp32 values as three bf16 parts each), each entry is an fp32 sum of m terms per 128-row chunk
(m = 128, or 9 * 128 part products for fp32 input) added across chunks in fp64, so
|G - X^T X| <= gamma_m (|X|^T |X|) elementwise, up to the fp64 sum.  A column of P then sits
within the Davis-Kahan angle sin(theta_i) <= ||E|| / (delta_i - ||E||) of the oracle's, with E
the Gram error (its Frobenius norm bounded by that of the elementwise bound) and delta_i the gap
from eigenvalue i to the rest of the spectrum (the eigenvalues taken as Rayleigh quotients of the
oracle's columns)."""
import numpy as np
import pytest
import torch

import sparse_dimension_attention_amd as aq
from oracle import aqua_oracle as O
from sparse_dimension_attention_amd.calibrate import calibrate_projection
from synth import make_projection, make_qk_block

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


def _stored(x64, dtype):
    t = torch.from_numpy(x64).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t, t.double().numpy()


def _gram_gpu(t):
    n, d = t.shape
    x = t.to(DEV)
    ws = torch.empty(aq.aqua_gram_workspace(aq.dtype_code(x.dtype), n, d), dtype=torch.uint8,
                     device=DEV)
    g = torch.empty(d, d, dtype=torch.float64, device=DEV)
    aq.aqua_gram(x, g, ws)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def _bound(X, dtype):
    m = 128 if dtype == "bf16" else 9 * 128
    gam = m * U / (1 - m * U)
    A = np.abs(X)
    # parts of an fp32 value: |h| + |m| + |l| <= |x| (1 + 2^-8 + 2^-16)
    scale = 1.0 if dtype == "bf16" else (1 + 2.0 ** -8 + 2.0 ** -16) ** 2
    return gam * scale * (A.T @ A) + 1e-13 * np.abs(X.T @ X).max()


@pytest.mark.parametrize("dtype,d,n", [
    ("bf16", 128, 1000),     # a ragged last chunk (104 rows)
    ("bf16", 64, 16384),     # 128 whole chunks
    ("f32", 128, 3000),
    ("f32", 64, 129),        # a last chunk of one row
])
def test_gram_matches_definition(dtype, d, n):
    rng = np.random.default_rng(21 + d + n)
    x64 = rng.standard_normal((n, d)) * np.exp(-np.arange(d) / 30.0) * 3.0
    t, X = _stored(x64, dtype)
    G = _gram_gpu(t)
    ref = X.T @ X  # fp64 sums of exact products: the definition to ~n 2^-53
    assert np.array_equal(G, G.T) or np.allclose(G, G.T, rtol=0, atol=_bound(X, dtype).max())
    assert np.all(np.abs(G - ref) <= _bound(X, dtype)), "Gram entry outside the fp32 bound"


def _check_projection(X, dtype, t, min_checked):
    P = calibrate_projection(t.to(DEV)).double().numpy()
    ref = O.calibrate(X)
    d = X.shape[1]
    assert np.allclose(P.T @ P, np.eye(d), atol=1e-6)
    lam = np.sum((X @ ref) ** 2, axis=0)  # Rayleigh quotients of the oracle's columns
    assert np.all(np.diff(lam) <= 1e-9 * lam[0])  # decreasing, as the oracle orders them
    E = np.linalg.norm(_bound(X, dtype))  # Frobenius norm of the elementwise bound
    checked = 0
    for i in range(d):
        others = np.delete(lam, i)
        gap = np.min(np.abs(others - lam[i]))
        if gap <= 2 * E:
            continue  # the bound says nothing about this column
        sin_bound = E / (gap - E) + 1e-9
        c = abs(float(P[:, i] @ ref[:, i]))
        sin_got = np.sqrt(max(0.0, 1.0 - c * c))
        assert sin_got <= sin_bound, (i, sin_got, sin_bound)
        # the sign rule picks the same sign once the columns are this close
        if sin_got < 0.1:
            assert P[:, i] @ ref[:, i] > 0, i
        checked += 1
    assert checked >= min_checked, f"only {checked} of {d} columns separated enough to check"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_calibrate_known_spectrum(dtype):
    """X = A diag(s) R^T with orthonormal A: X^T X = R diag(s^2) R^T, s evenly spaced from 40
    down to 20, so that every column's gap (>= 12.7) exceeds twice the Gram error bound (0.3 for
    bf16, 2.7 for fp32 input): all 64 columns are checked."""
    d, n = 64, 4096
    rng = np.random.default_rng(31)
    A = np.linalg.qr(rng.standard_normal((n, d)))[0]
    R = np.linalg.qr(rng.standard_normal((d, d)))[0]
    s = 40.0 * (1 - np.arange(d) / (2 * d))
    t, X = _stored((A * s) @ R.T, dtype)
    _check_projection(X, dtype, t, min_checked=d)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_calibrate_generator_vectors(dtype):
    """The generator's query and key vectors (the retention study's calibration set)."""
    P64 = make_projection(2, 128)
    q, _ = make_qk_block(2, "calib_q", (0, 0), 4096, 128, 40.0, P64)
    k, _ = make_qk_block(2, "calib_k", (0, 0), 4096, 128, 40.0, P64)
    t, X = _stored(np.concatenate([q, k]), dtype)
    _check_projection(X, dtype, t, min_checked=8)
