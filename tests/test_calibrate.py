"""The host half of the offline projection (the eigensolve of a Gram matrix) against the oracle's
calibration (CPU; the Gram matrix here is the definition X^T X in fp64; the GPU's Gram matrix is
checked in test_gpu_calibrate.py)."""
import numpy as np
import torch

from oracle import aqua_oracle as O
from sparse_dimension_attention_amd.calibrate import projection_from_gram
from synth import make_projection, make_qk_block


def _check(X):
    P = projection_from_gram(torch.from_numpy(X.T @ X)).double().numpy()
    ref = O.calibrate(X)
    n, d = X.shape
    r = min(n, d)  # past the samples' rank the directions are any basis of what they miss
    assert P.shape == ref.shape == (d, d)
    assert np.allclose(P[:, :r], ref[:, :r], atol=2e-6)
    assert np.allclose(P.T @ P, np.eye(d), atol=1e-6)
    assert np.max(np.abs(X @ P[:, r:]), initial=0.0) < 1e-5 * np.max(np.abs(X))


def test_calibrate_matches_oracle_random():
    rng = np.random.default_rng(5)
    _check(rng.standard_normal((300, 24)) * np.exp(-np.arange(24) / 5.0))


def test_calibrate_matches_oracle_fewer_samples_than_dims():
    rng = np.random.default_rng(6)
    _check(rng.standard_normal((7, 16)) * np.exp(-np.arange(16) / 3.0))


def test_calibrate_matches_oracle_generator():
    P64 = make_projection(2, 128)
    q, _ = make_qk_block(2, "calib_q", (0, 0), 4096, 128, 40.0, P64)
    k, _ = make_qk_block(2, "calib_k", (0, 0), 4096, 128, 40.0, P64)
    _check(np.concatenate([q, k]))
