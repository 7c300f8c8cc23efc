"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic (no RoPE, no softmax, no projection, no merge).  Both the
fp64 oracle and the HIP path receive exactly the arrays produced here.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    TensorId,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    normal_bf16,
    kv_raw,
    query,
    ragged_lengths,
    paged_table,
    workload,
)
