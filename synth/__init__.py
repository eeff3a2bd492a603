"""Seeded synthetic inputs for the Ulysses H3 hot path.

This package holds no arithmetic of the method: it only draws random numbers
and segment lengths and describes the workload shapes.  It is the one module
that both the fp64 oracle's tests and the HIP path's tests and bench read.
"""
from .workloads import WORKLOADS, Workload, segment_offsets  # noqa: F401
from .inputs import normal_bf16, normal_bf16_bits, unique_pattern_bits  # noqa: F401
