"""Seeded synthetic inputs for the QSA layer path.

This package only draws inputs (index keys, index queries, Q/K/V, query-row
positions, segment cut points). It performs none of the method's arithmetic
(no pooling, scoring, selection or attention), so both the CPU oracle and the
HIP path may import it without sharing any computation.
"""
from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    SeqSpec,
    bf16_bits,
    round_bf16,
    gen_layer,
    gen_batched_layer,
    batched_specs,
    fill_layer_device,
    planting_direction,
)
