"""Seeded synthetic inputs for the CSA2 hot path.

This package draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, scoring, selection or attention).  Both
the oracle-based tests and the GPU path take their inputs from here.
"""
from .workloads import (  # noqa: F401
    Layer, Workload, WORKLOADS, workload, f32_to_bf16_bits, bf16_bits_to_f32,
    SequenceData, QueryData, gen_sequence, gen_batch, gen_queries, gen_structure,
)
