"""Seeded synthetic workloads for the low-bit recurrent-state decode step.

This package holds the five workload configurations and the seeded input
generators. It is the only code shared by the CPU oracle and the GPU path,
and it contains none of the method's arithmetic: no decay, no update, no
quantizer. It only draws the per-step inputs (q, k, v and the gates) from the
distributions each workload names, and rounds them to the input dtype.

The recurrence the inputs feed is the one in Table 1 of "Preserving Updates in
Low-Bit Recurrent State Quantization" (decay A_t and update B_t for RetNet,
Mamba2, GLA and Gated DeltaNet).
"""
from .configs import CONFIGS, Workload, head_bits_for
from .gen import bf16_round, step_inputs, static_params, InputPool

__all__ = ["CONFIGS", "Workload", "head_bits_for", "bf16_round",
           "step_inputs", "static_params", "InputPool"]
