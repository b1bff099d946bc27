"""Seeded synthetic decode-attention workloads.

This package only draws random inputs; it holds none of the method's arithmetic
(no quantizer, no ranking, no attention).  Both the CPU oracle and the HIP path
take their inputs from here, so that a parity test compares the two on exactly
the same tensors.
"""
from .configs import CONFIGS, WorkloadConfig, get_config
from .gen import (SliceInputs, generate_slice, generate_query, generate_all, planted_positions,
                  generate_step_queries)

__all__ = [
    "CONFIGS", "WorkloadConfig", "get_config",
    "SliceInputs", "generate_slice", "generate_query", "generate_all", "planted_positions",
    "generate_step_queries",
]
