"""Seeded synthetic inputs for the sparse-attention hot path.

This package only *makes inputs*: shapes, random draws, the structure the
workloads call for (outlier channels, positional drift, planted needle blocks)
and the one-time rounding of fp32 draws to bf16 storage bits.  It holds none of
the method's arithmetic (no sketches, scores, selections or attention); both
the CPU oracle and the GPU path consume the arrays it returns.
"""
from .configs import WORKLOADS, Workload, get_workload
from .generate import (DecodeInputs, PrefillInputs, bf16_bits_to_f32,
                       f32_to_bf16_bits, make_decode_inputs,
                       make_prefill_inputs, make_inputs)

__all__ = [
    "WORKLOADS", "Workload", "get_workload", "DecodeInputs", "PrefillInputs",
    "bf16_bits_to_f32", "f32_to_bf16_bits", "make_decode_inputs",
    "make_prefill_inputs", "make_inputs",
]
