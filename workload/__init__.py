"""Seeded synthetic workloads for the rotated INT2 KV cache (inputs only).

This package draws random keys, values, queries, rotations, context lengths and
block tables. It holds none of the method's arithmetic (no centring, rotation,
quantisation or attention); both the float64 oracle and the HIP path consume
what it produces.
"""
from .gen import (  # noqa: F401
    EXPM_SCALE,
    WORKLOADS,
    Workload,
    block_table_for,
    corrected_rotation,
    ctx_lens_for,
    haar_orthogonal,
    hadamard,
    kv_for_sequence,
    make_static,
    query_for,
    key_mean,
    scaled,
)
