"""CPU oracle for Q4_0 (test infrastructure only; see ``q4_0``)."""

from .q4_0 import (  # noqa: F401
    QK,
    BLOCK_BYTES,
    packed_size,
    widen_bf16,
    quantize,
    unpack,
    dequantize,
    matmul_ref,
    tolerance,
    check,
    TOL_REL,
    TOL_ABS,
)
