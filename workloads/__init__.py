"""Seeded synthetic inputs for the paged decode-attention workloads.

This package draws random numbers and fixes shapes; it holds none of the
method's arithmetic (no block allocation, no slot computation, no cache
layout, no attention).  Both the CPU oracle and the GPU path take their
inputs from here and from nowhere else.
"""
from .synth import SPECS, Workload, WorkloadSpec, generate, spec, round_bf16_bits, bf16_bits_to_f32

__all__ = ["SPECS", "Workload", "WorkloadSpec", "generate", "spec",
           "round_bf16_bits", "bf16_bits_to_f32"]
