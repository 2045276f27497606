"""Seeded synthetic inputs for the block-sparse prefill path.

This package only draws random numbers and encodes them into the storage
formats the path consumes (bf16 bit patterns, OCP e4m3 codes with per-head
scales, fp32).  It holds none of the method's arithmetic, and it is the one
module that both the fp64 oracle tests and the GPU path import.
"""

from .workloads import (  # noqa: F401
    ALPHA_SWEEP,
    CONFIGS,
    Workload,
    WorkloadSpec,
    chunk_view,
    make_workload,
    spec_for,
    custom_spec,
)
