"""Seeded synthetic inputs for the ReSpinQuant online path.

This package holds only random draws and the fixed workload shapes. It
computes none of the method: no rotation, no basis-mismatch matrix, no
subspace, no normalisation and no quantisation. Both the CPU oracle and the
GPU path read their inputs from here, and from nothing else they share.
"""
from .workloads import (
    WORKLOADS, Workload, Linear, layer_linears, workload,
    TINY, LLAMA2_7B_PREFILL, LLAMA2_7B_DECODE, LLAMA3_8B_W3A3, LLAMA2_70B_PREFILL,
)
from .generators import (
    residual,
    skew_generator,
    low_rank_skew,
    weight,
    linear_input,
    outlier_channels,
    to_bf16_bits,
    bf16_bits_to_f32,
)

__all__ = [
    "WORKLOADS", "Workload", "Linear", "layer_linears", "workload",
    "TINY", "LLAMA2_7B_PREFILL", "LLAMA2_7B_DECODE", "LLAMA3_8B_W3A3", "LLAMA2_70B_PREFILL",
    "residual", "skew_generator", "low_rank_skew", "weight", "linear_input", "outlier_channels",
    "to_bf16_bits", "bf16_bits_to_f32",
]
