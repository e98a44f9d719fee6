"""Seeded synthetic inputs for AQUA attention (shared by the oracle's tests and the HIP path).

This module only draws and stores input tensors.  It contains none of the method's arithmetic:
no projection of queries or keys by P for the method, no selection, no attention.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    config,
    decay,
    make_projection,
    make_qk_block,
    make_v_block,
    to_storage,
    storage_to_f64,
    make_decode_inputs,
    make_prefill_inputs,
    make_h2o_inputs,
    rng_for,
)
