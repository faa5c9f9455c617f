"""Seeded synthetic workloads for the rank-augmented W4A4 linear layer.

Only random draws and their layout live here; none of the layer's arithmetic
(quantisation, integer product, epilogue) does.  Both the CPU oracle's tests
and the GPU path's tests and benchmark take their inputs from this package.
"""

from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    draw_linear,
    draw_custom,
    draw_group,
    draw_group_custom,
    draw_two_subspace,
    draw_two_subspace_custom,
    to_bf16_values,
)
