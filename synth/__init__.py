"""Seeded synthetic inputs for the quantized MoE feed-forward layer.

This package is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It draws random numbers and lays them out in the
canonical block formats; it contains none of the layer's arithmetic (no
dequantization, no dot products, no routing, no activation).
"""

from .formats import (  # noqa: F401
    FORMATS, QMatrix, row_bytes, matrix_bytes, blocks_per_row,
    pack_q8_0, pack_q4_0, pack_i8_row, pack_i4_row, f32_to_bf16_bits,
)
from .workloads import (  # noqa: F401
    MoESpec, DenseSpec, SPECS, spec, moe_router, moe_expert, moe_shared, moe_x,
    moe_expert_stack, dense_matrix, dense_x,
)
