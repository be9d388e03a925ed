"""Helpers for the GPU parity tests: moving the seeded bf16 inputs to the
device, and a cache of oracle results so each large tensor is quantised
on the CPU once per session."""
import os

import numpy as np
import torch

import oracle
from workloads import tensor_bits, x_bits, workload

THREADS = min(16, os.cpu_count() or 1)
_cache = {}


def dev():
    return torch.device("cuda:0")


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(dev())


def gpu_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def weight_bits(wl: str, name: str) -> np.ndarray:
    key = ("W", wl, name)
    if key not in _cache:
        _cache[key] = tensor_bits(workload(wl).tensor(name))
    return _cache[key]


def act_bits(wl: str, name: str) -> np.ndarray:
    key = ("x", wl, name)
    if key not in _cache:
        _cache[key] = x_bits(workload(wl).x(name))
    return _cache[key]


def oracle_quant(wl: str, name: str):
    key = ("Q", wl, name)
    if key not in _cache:
        _cache[key] = oracle.quantize(weight_bits(wl, name))
    return _cache[key]


def assert_within_tolerance(y_gpu, y_ref, l1, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), what
    ok, worst = oracle.tolerance_ok(y_gpu, y_ref, l1)
    assert ok, "%s: |y_gpu - y_ref| exceeds 2e-3*sum|w*x| (worst ratio %.3g)" % (what, worst)
    return worst
