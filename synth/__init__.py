"""Seeded synthetic inputs for the fused per-state norm + FC step.

This package only *draws* inputs: hidden states, norm parameters, the FC
weight and bias, rounded to bfloat16.  It holds none of the method's
arithmetic (no statistics, no normalisation, no matmul), so both the fp64
oracle and the HIP path can read the same bits from it without sharing any
computation.
"""

from .workloads import CONFIGS, Workload, workload
from .gen import Inputs, make_inputs, make_embed_inputs, bf16_round, bf16_bits, bits_to_f32
from .verify import make_verify_inputs

__all__ = [
    "CONFIGS",
    "Workload",
    "workload",
    "Inputs",
    "make_inputs",
    "make_embed_inputs",
    "make_verify_inputs",
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
]
