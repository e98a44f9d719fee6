"""Offline projection for AQUA: P from an SVD of calibration vectors.

The method's first, offline phase (digest of arXiv 2509.11155, section 方法详解 / 技术框架: the
projection is learned once by SVD on a calibration set; edgentiq blog, "How AQUA Works", step 1).
It runs once before any decoding and is not part of the online step.  The O(n d^2) work, the Gram
matrix G = X^T X of the calibration vectors, is libaqua's (aqua_gram, on the GPU); the d x d
symmetric eigensolve of G is left on the host (float64): P's columns are G's eigenvectors, which
are X's right singular vectors.

Readings where the pages say no more than "SVD on a calibration dataset": the calibration set is
the stacked query and key vectors of one head group; P's columns are the right singular vectors
in decreasing order of singular value, so that dim i of q' = q P is the i-th most important
direction (the order AQUA-Memory's static cut keeps); the sign the SVD leaves free is fixed per
column so that its entry of largest magnitude is positive.
"""
from __future__ import annotations

import torch

from . import aqua as _aq


def projection_from_gram(gram: torch.Tensor) -> torch.Tensor:
    """P [d][d] float32 (host) from the Gram matrix G = X^T X [d][d] of the calibration vectors:
    G's eigenvectors in decreasing order of eigenvalue, each column's sign fixed so that its
    entry of largest magnitude is positive.  A rank-deficient G (fewer samples than dims) still
    gives d orthonormal columns: past the rank, a basis of the directions the samples miss."""
    g = gram.detach().to("cpu", torch.float64)
    d = g.shape[0]
    w, v = torch.linalg.eigh(0.5 * (g + g.transpose(0, 1)))
    v = v.flip(1)  # decreasing eigenvalue
    lead = v.abs().argmax(dim=0)
    sign = torch.sign(v[lead, torch.arange(d)])
    return (v * sign).to(torch.float32).contiguous()


def calibrate_projection(samples: torch.Tensor, stream=None) -> torch.Tensor:
    """P [d][d] float32 (host) from calibration vectors `samples` [n][d] (bf16 or float32, on the
    GPU): G = X^T X by aqua_gram, then projection_from_gram."""
    if samples.ndim != 2:
        raise ValueError(f"samples must be [n][d], got shape {tuple(samples.shape)}")
    if not samples.is_cuda:
        raise ValueError("calibration vectors must be on the GPU (libaqua computes their Gram "
                         "matrix there)")
    x = samples.contiguous()
    n, d = x.shape
    ws = torch.empty(_aq.aqua_gram_workspace(_aq.dtype_code(x.dtype), n, d), dtype=torch.uint8,
                     device=x.device)
    gram = torch.empty(d, d, dtype=torch.float64, device=x.device)
    _aq.aqua_gram(x, gram, ws, stream)
    return projection_from_gram(gram)
