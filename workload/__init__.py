"""Seeded synthetic workloads for the MLA gather-decode step.

This package only draws inputs (weights, activations, index tensors, the paged
cache pool).  It holds none of the step's arithmetic, so both the fp64 oracle
and the GPU path can be fed from it without sharing any method code.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    ROUTER_CONFIGS,
    make_router_inputs,
    MlaShape,
    Workload,
    config_by_name,
    fill_pool_,
    make_inputs,
    pool_rows,
    splitmix64_np,
    splitmix64_torch,
    to_device,
)
