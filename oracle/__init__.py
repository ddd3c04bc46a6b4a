"""CPU oracle for the low-bit recurrent-state decode step.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or run anything in this package. The
product path (the HIP library and its Python binding) never calls it, and the
two share no code: the oracle is numpy only and is written from the pages'
definitions.

What it computes (one step of one or many (batch, head) state tiles):
  * the recurrence S_t = A_t S_{t-1} + B_t with the four rows of Table 1 of
    "Preserving Updates in Low-Bit Recurrent State Quantization"
    (RetNet gamma*I / k v^T, Mamba2 alpha_t*I / k v^T,
    GLA Diag(alpha_t) / k v^T, Gated DeltaNet alpha_t*I /
    beta_t k (v - (A_t S_{t-1})^T k)^T);
  * the readout o_t = S_t^T q_t;
  * group-wise symmetric requantization after every update (abstracts of
    "Preserving Updates ..." and "When Dynamic Scaling Fails ..."), with
    dynamic, persistent or reference-yoked scales (the latter two from the
    abstract of "When Dynamic Scaling Fails ...");
  * Bounded Directional Rounding and the Low-Rank Bypass with its periodic
    merge ("Preserving Updates ...", abstract, Fig. 3, Fig. 4, Table 6).

Arithmetic runs in one of two modes:
  'f32'  the canonical fp32 chain: every operation rounds to float32 in the
         order written here, fused multiply-adds are emulated exactly. This is
         the mode the GPU path is compared with, code for code.
  'f64'  definitional: the same algorithm in float64 (storage roundings of
         scales, inputs and bypass factors still apply). Pins use this mode.

Parity status: the floating-point chain order (which operations fuse, and
the pairwise order of the Gated DeltaNet retrieval sum) is a reading, not
something the pages fix; see each function. Where a function has no
independent pin it says "parity unpinned".
"""
from .fp import F32, F64, Arith, fma32, pairwise_sum, f16_round, f16_of_exact
from .recurrence import (OState, zero_state, step, merge, readout, decay_rows,
                         scale_rule, quantize_group_codes, qrange)
from . import closed_form, brute, accounting, allocation, diagnostics, hadamard, window

__all__ = ["F32", "F64", "Arith", "fma32", "pairwise_sum", "f16_round",
           "OState", "zero_state", "step", "merge", "readout", "decay_rows",
           "scale_rule", "quantize_group_codes", "qrange",
           "closed_form", "brute", "accounting", "allocation", "diagnostics", "hadamard", "window"]
