"""Synthetic workloads for the RaggedShard/DBuffer layout transform.

This package only describes inputs: tensor shapes, atomic-block kinds, rank
counts, value distributions and seeded generators. It holds none of the
method's arithmetic (no granularities, plans, scaling or quantisation), so
both the CPU oracle and the HIP path can take their inputs from it without
sharing any of the computation.
"""
from .configs import (TensorSpec, Workload, WORKLOADS, adam_tile32_variant, workload, tiny_variant,
                      tile_major_variant)
from .gen import (
    Role,
    seed_key,
    normal_f32,
    uniform_f32,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    draw,
    tensor_values,
    weight_bits,
    prev_slice,
    adam_state,
    parallel_map,
    worker_count,
)

__all__ = [
    "TensorSpec", "Workload", "WORKLOADS", "workload", "tiny_variant", "tile_major_variant", "adam_tile32_variant",
    "Role", "seed_key", "normal_f32", "uniform_f32", "bf16_bits_from_f32",
    "f32_from_bf16_bits", "draw", "tensor_values", "weight_bits", "prev_slice",
    "adam_state", "parallel_map", "worker_count",
]
