"""Offline projection for AQUA: P from an SVD of calibration vectors.

The method's first, offline phase (digest of arXiv 2509.11155, section 方法详解 / 技术框架: the
projection is learned once by SVD on a calibration set; edgentiq blog, "How AQUA Works", step 1).
It runs once on the host before any decoding and is not part of the online step that libaqua
implements; it uses a library SVD in float64.

Readings where the pages say no more than "SVD on a calibration dataset": the calibration set is
the stacked query and key vectors of one head group; P's columns are the right singular vectors
in decreasing order of singular value, so that dim i of q' = q P is the i-th most important
direction (the order AQUA-Memory's static cut keeps); the sign the SVD leaves free is fixed per
column so that its entry of largest magnitude is positive.
"""
from __future__ import annotations

import torch


def calibrate_projection(samples: torch.Tensor) -> torch.Tensor:
    """P [d][d] float32 (on the host) from calibration vectors `samples` [N][d], any float dtype
    and device; computed in float64."""
    if samples.ndim != 2:
        raise ValueError(f"samples must be [N][d], got shape {tuple(samples.shape)}")
    x = samples.detach().to("cpu", torch.float64)
    n, d = x.shape
    # all d right singular vectors; with fewer samples than dims the full factorisation supplies
    # the directions the samples do not reach
    v = torch.linalg.svd(x, full_matrices=n < d).Vh.transpose(0, 1)
    lead = v.abs().argmax(dim=0)
    sign = torch.sign(v[lead, torch.arange(d)])
    return (v * sign).to(torch.float32).contiguous()
