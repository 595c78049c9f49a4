"""Seeded synthetic inputs for the Q4_0 linear layer.

This package only draws numbers: weight matrices, activation batches and the
edge-case blocks used by the tests.  It holds none of the quantisation or
matmul arithmetic, so both the CPU oracle and the HIP library can be fed from
it without sharing any of the method's code.
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    Linear,
    rng_for,
    normal_weights,
    outlier_weights,
    student_t_weights,
    workload_weights,
    workload_activations,
    random_weights,
    random_activations,
    bf16_bits,
    edge_case_weights,
    sha256_of,
)
