"""Counter-based seeded generator for bf16 test tensors.

Element ``i`` of a stream with seed ``s`` is a pure function of ``(s, i)``,
so any slice of a tensor can be regenerated without drawing the rest.

* Uniform bits: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014), in its counter form: the
  i-th output of the generator seeded with ``s`` mixes ``s + (i+1)*gamma``
  with gamma = 0x9E3779B97F4A7C15 and the published finaliser constants.
* Uniform [0,1): the top 53 bits of an output times 2**-53.
* Normal: Box-Muller (G. Box, M. Muller, 1958). Element ``i`` uses outputs
  ``2i`` and ``2i+1``: z = sqrt(-2 ln(1-u0)) * cos(2*pi*u1), in float64.
* Outliers: element ``i`` is scaled by ``outlier_scale`` when output ``i`` of
  a second stream (seed ``s ^ OUTLIER_SALT``) gives a uniform below
  ``outlier_p`` (independent Bernoulli draws), before rounding.
* Rounding: sigma*z (float64) -> float32 (round to nearest even, numpy's
  cast) -> bfloat16 (round to nearest even on the float32 bits).

The result is returned as raw uint16 bfloat16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
MIX1 = np.uint64(0xBF58476D1CE4E5B9)
MIX2 = np.uint64(0x94D049BB133111EB)
OUTLIER_SALT = 0x5DEECE66D
_CHUNK = 1 << 23


def splitmix64(seed: int, index: np.ndarray) -> np.ndarray:
    """Output ``index`` (uint64 array, 0-based) of the SplitMix64 stream ``seed``."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (index.astype(np.uint64) + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * MIX1
        z = (z ^ (z >> np.uint64(27))) * MIX2
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, index: np.ndarray) -> np.ndarray:
    """float64 uniforms in [0, 1) from the top 53 bits of each output."""
    return (splitmix64(seed, index) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(seed: int, start: int, count: int) -> np.ndarray:
    """float64 standard normals for elements ``start .. start+count-1``."""
    i = np.arange(start, start + count, dtype=np.uint64)
    u0 = uniform01(seed, np.uint64(2) * i)
    u1 = uniform01(seed, np.uint64(2) * i + np.uint64(1))
    return np.sqrt(-2.0 * np.log1p(-u0)) * np.cos(2.0 * np.pi * u1)


def float32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the generator never produces inf or nan)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_float32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_tensor_numpy(shape, seed: int, sigma: float, start: int = 0,
                      outlier_p: float = 0.0, outlier_scale: float = 1.0) -> np.ndarray:
    """numpy version of ``bf16_tensor`` (slow; used to cross-check the C version).

    Elements are numbered row-major from ``start`` within the stream ``seed``.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        v = normal(seed, start + c0, c1 - c0) * sigma
        if outlier_p > 0.0:
            idx = np.arange(start + c0, start + c1, dtype=np.uint64)
            hit = uniform01(seed ^ OUTLIER_SALT, idx) < outlier_p
            v[hit] *= outlier_scale
        out[c0:c1] = float32_to_bf16_bits(v.astype(np.float32))
    return out.reshape(shape)


_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libwlgen.so")
_lib = None


def build_native(force: bool = False) -> str:
    """Compile gen.c into libwlgen.so next to it (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
                               os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _native():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_native())
        lib.wl_gen_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int64,
                                    ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int]
        lib.wl_gen_bf16.restype = None
        lib.wl_splitmix64.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int64]
        lib.wl_splitmix64.restype = None
        _lib = lib
    return _lib


def splitmix64_native(seed: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _native().wl_splitmix64(out.ctypes.data, count, seed & 0xFFFFFFFFFFFFFFFF, start)
    return out


def bf16_tensor(shape, seed: int, sigma: float, start: int = 0,
                outlier_p: float = 0.0, outlier_scale: float = 1.0, threads: int = 0) -> np.ndarray:
    """A bf16 tensor (uint16 bits) of ``shape`` drawn as sigma*N(0,1).

    Elements are numbered row-major from ``start`` within the stream ``seed``.
    The bits are independent of ``threads``.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    nt = threads or min(16, os.cpu_count() or 1)
    _native().wl_gen_bf16(out.ctypes.data, n, seed & 0xFFFFFFFFFFFFFFFF, start, float(sigma),
                          float(outlier_p), float(outlier_scale), nt)
    return out.reshape(shape)


def fp8_release(shape, seed: int, sigma: float, outlier_p: float = 0.0, outlier_scale: float = 1.0):
    """A synthetic weight tensor as a checkpoint released in FP8 holds it: the
    seeded sigma*N(0,1) weights of ``bf16_tensor`` (as fp32), one fp32 scale
    per tensor that maps the largest magnitude onto E4M3's largest finite
    value (448), and weight / scale cast to OCP E4M3 ("fn") by torch
    (nearest-even, clipped to +-448). Returns (codes uint8 ``shape``, scale
    np.float32)."""
    import torch

    w = bf16_to_float32(bf16_tensor(shape, seed, sigma, outlier_p=outlier_p, outlier_scale=outlier_scale))
    amax = float(np.abs(w).max())
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    q = np.clip(w / scale, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def norm_gain(K: int, seed: int, sigma: float = 0.1) -> np.ndarray:
    """A synthetic RMS-norm gain vector (uint16 bf16 bits, length ``K``): 1 +
    sigma*N(0,1) with the normal draws of ``bf16_tensor`` (seed ``seed``),
    the sum rounded once to bf16 (nearest even), the shape of a trained
    norm's gains around one."""
    g = 1.0 + bf16_to_float32(bf16_tensor((K,), seed, sigma)).astype(np.float64)
    return float32_to_bf16_bits(g.astype(np.float32))
