"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds only input generation (random bf16 tensors, their FP8
release form, and the workload shape table). It contains none of the NVFP4 arithmetic, so that the
oracle and the GPU path can both consume the same bits without sharing code.
"""
from .gen import (splitmix64, uniform01, normal, bf16_tensor, bf16_tensor_numpy, bf16_to_float32,
                  float32_to_bf16_bits, build_native, fp8_release, norm_gain)
from .configs import WORKLOADS, Tensor, Workload, workload, tensor_bits, x_bits

__all__ = [
    "splitmix64", "uniform01", "normal", "bf16_tensor", "bf16_tensor_numpy", "bf16_to_float32",
    "float32_to_bf16_bits", "build_native", "fp8_release", "norm_gain",
    "WORKLOADS", "Tensor", "Workload", "workload", "tensor_bits", "x_bits",
]
