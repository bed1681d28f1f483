"""Seeded synthetic inputs shaped like the workloads of the DB-SpMSpV paper.

This package only draws inputs (matrices in CSR form, sparse and dense
vectors).  It holds none of the SpMSpV arithmetic: both the CPU oracle and the
HIP library consume what it produces, and neither is imported here.
"""
from .generators import (  # noqa: F401
    rng_for,
    uniform_csr,
    rmat_csr,
    permute_vertices,
    largest_component_vertices,
    decode_weight_csr,
    decode_activation,
    zipf_band_csr,
    sparse_x,
    sparse_x_with_dense_blocks,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    csr_from_dense,
)
