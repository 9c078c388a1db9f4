"""Seeded synthetic inputs for the five MoE dispatch/combine workloads.

This module only draws random inputs and stores them in the formats the path
consumes (fp32, bfloat16 bit patterns, fp8 E4M3FN bit patterns with
per-128-element fp32 block scales).  It holds none of the routing, dispatch or
combine arithmetic, so both the CPU oracle and the HIP path can use it.
"""
from .gen import (CONFIGS, DECODE_FFN, FP8_GEMM_N, WorkloadConfig, alternating_sort, make_fp8_expert_weights_device,
                  make_inputs, make_swiglu_weights, make_swiglu_weights_device)

__all__ = ["CONFIGS", "DECODE_FFN", "FP8_GEMM_N", "WorkloadConfig", "make_inputs", "make_swiglu_weights",
           "make_swiglu_weights_device", "make_fp8_expert_weights_device", "alternating_sort"]
