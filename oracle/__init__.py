"""NVFP4 oracle (TEST INFRASTRUCTURE ONLY).

A plain CPU implementation in C (``nvfp4_oracle.c``): table decode of E2M1 and
E4M3, the fp32 quantisation rule step by step, and the product accumulated in
fp64. Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the GPU library never uses it.

Functions take and return numpy arrays; bf16 tensors are uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

# gcc, -O2, strict IEEE: no fast-math, no contraction of a*b+c into fma.
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-std=c99"]


def build(force: bool = True) -> str:
    """Compile the oracle into liboracle.so next to its source."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


# Test hook: the planted-mistake tests point this at a deliberately broken
# build of the same source, to show that the pins catch each mistake.
_OVERRIDE_ENV = "ORACLE_LIBRARY_OVERRIDE"


def _L():
    global _lib
    if _lib is None:
        path = os.environ.get(_OVERRIDE_ENV) or _SO
        if path == _SO and not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(path)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.orc_e2m1_value.argtypes = [ctypes.c_int]
        lib.orc_e2m1_value.restype = ctypes.c_double
        lib.orc_e4m3_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e2m1_encode.argtypes = [ctypes.c_float]
        lib.orc_e2m1_encode.restype = ctypes.c_uint8
        lib.orc_quantize.argtypes = [P, I64, I64, P, P, P]
        lib.orc_quantize.restype = ctypes.c_int
        lib.orc_quantize_fp8.argtypes = [P, ctypes.c_float, I64, I64, P, P, P]
        lib.orc_quantize_fp8.restype = ctypes.c_int
        lib.orc_quantize_f32.argtypes = [P, I64, I64, P, P, P]
        lib.orc_quantize_f32.restype = ctypes.c_int
        lib.orc_dequant.argtypes = [P, P, ctypes.c_float, I64, I64, P]
        lib.orc_dequant.restype = None
        lib.orc_gemv.argtypes = [P, I64, P, P, ctypes.c_float, I64, I64, P, P, ctypes.c_int]
        lib.orc_gemv.restype = None
        lib.orc_tile.argtypes = [P, P, I64, I64, P]
        lib.orc_tile.restype = None
        lib.orc_e4m3_encode_n.argtypes = [P, I64, P]
        lib.orc_e4m3_encode_n.restype = None
        lib.orc_e2m1_encode_n.argtypes = [P, I64, P]
        lib.orc_e2m1_encode_n.restype = None
        lib.orc_gemv_f64.argtypes = [P, I64, P, P, ctypes.c_float, I64, I64, P, P, ctypes.c_int]
        lib.orc_gemv_f64.restype = None
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_swiglu.argtypes = [P, P, I64, P]
        lib.orc_swiglu.restype = None
        lib.orc_rmsnorm.argtypes = [P, P, I64, I64, ctypes.c_double, P]
        lib.orc_rmsnorm.restype = None
        lib.orc_e8m0_value.argtypes = [ctypes.c_int]
        lib.orc_e8m0_value.restype = ctypes.c_double
        lib.orc_mx_quantize.argtypes = [P, I64, I64, P, P]
        lib.orc_mx_quantize.restype = ctypes.c_int
        lib.orc_mx_dequant.argtypes = [P, P, I64, I64, P]
        lib.orc_mx_dequant.restype = None
        lib.orc_mx_gemv.argtypes = [P, I64, P, P, I64, I64, P, P]
        lib.orc_mx_gemv.restype = None
        lib.orc_mx_tile.argtypes = [P, P, I64, I64, P]
        lib.orc_mx_tile.restype = None
        for f in (lib.orc_argmax_rows_f64, lib.orc_argmax_rows_f32):
            f.argtypes = [P, I64, I64, I64, P]
            f.restype = None
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def e2m1_value(code: int) -> float:
    return _L().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return _L().orc_e4m3_value(int(code))


def e4m3_encode(s: float) -> int:
    return int(_L().orc_e4m3_encode(float(s)))


def e2m1_encode(v: float) -> int:
    return int(_L().orc_e2m1_encode(float(v)))


def e4m3_encode_array(s: np.ndarray) -> np.ndarray:
    a, pa = _c(np.ravel(s), np.float32)
    out = np.empty(a.size, dtype=np.uint8)
    _L().orc_e4m3_encode_n(pa, a.size, out.ctypes.data)
    return out


def e2m1_encode_array(v: np.ndarray) -> np.ndarray:
    a, pa = _c(np.ravel(v), np.float32)
    out = np.empty(a.size, dtype=np.uint8)
    _L().orc_e2m1_encode_n(pa, a.size, out.ctypes.data)
    return out


def quantize(W_bits: np.ndarray):
    """W (uint16 bf16 bits [N][K]) -> (packed uint8 [N][K/2], scales uint8 [N][K/16], gscale float32)."""
    W, pw = _c(W_bits, np.uint16)
    N, K = W.shape
    packed = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    rc = _L().orc_quantize(pw, N, K, packed.ctypes.data, scales.ctypes.data, g.ctypes.data)
    if rc != 0:
        raise ValueError("orc_quantize: bad shape %r" % (W.shape,))
    return packed, scales, np.float32(g[0])


def _quantize_with(fn, W: np.ndarray, ptr, *lead):
    N, K = W.shape
    packed = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    rc = fn(ptr, *lead, N, K, packed.ctypes.data, scales.ctypes.data, g.ctypes.data)
    if rc != 0:
        raise ValueError("quantize: bad shape %r" % (W.shape,))
    return packed, scales, np.float32(g[0])


def quantize_fp8(W_codes: np.ndarray, scale) -> tuple:
    """FP8 E4M3 codes (uint8 [N][K]) with one fp32 dequantisation scale: the
    element values E4M3(code) * scale (one fp32 rounding) go through the same
    rule as quantize(). Returns (packed, scales, gscale)."""
    W, pw = _c(W_codes, np.uint8)
    L = _L()
    return _quantize_with(lambda p, *a: L.orc_quantize_fp8(p, float(np.float32(scale)), *a), W, pw)


def quantize_f32(W: np.ndarray) -> tuple:
    """fp32 values [N][K] through the same rule as quantize()."""
    W, pw = _c(W, np.float32)
    return _quantize_with(_L().orc_quantize_f32, W, pw)


def dequant(packed: np.ndarray, scales: np.ndarray, gscale) -> np.ndarray:
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    N, K = packed.shape[0], packed.shape[1] * 2
    out = np.empty((N, K), dtype=np.float64)
    _L().orc_dequant(pp, ps, float(np.float32(gscale)), N, K, out.ctypes.data)
    return out


def gemv(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, gscale, threads: int = 1,
         with_l1: bool = True):
    """fp64 product y[M][N] (and the error scale l1[M][N]) for bf16 x [M][K]."""
    x, px = _c(np.atleast_2d(x_bits), np.uint16)
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    M, K = x.shape
    N = packed.shape[0]
    assert packed.shape[1] * 2 == K and scales.shape == (N, K // 16)
    y = np.empty((M, N), dtype=np.float64)
    l1 = np.empty((M, N), dtype=np.float64) if with_l1 else None
    _L().orc_gemv(px, M, pp, ps, float(np.float32(gscale)), N, K, y.ctypes.data,
                  l1.ctypes.data if with_l1 else None, int(threads))
    return (y, l1) if with_l1 else y


def gemv_f64(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, gscale, threads: int = 1):
    """The product for fp64 activations x [M][K] (e.g. RMS-normalised rows):
    (y [M][N], l1 [M][N]) as gemv()."""
    x, px = _c(np.atleast_2d(x), np.float64)
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    M, K = x.shape
    N = packed.shape[0]
    assert packed.shape[1] * 2 == K and scales.shape == (N, K // 16)
    y = np.empty((M, N), dtype=np.float64)
    l1 = np.empty((M, N), dtype=np.float64)
    _L().orc_gemv_f64(px, M, pp, ps, float(np.float32(gscale)), N, K, y.ctypes.data, l1.ctypes.data, int(threads))
    return y, l1


def silu(z: float) -> float:
    return _L().orc_silu(float(z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u elementwise, fp64 (g: gate product, u: up product)."""
    g, pg = _c(g, np.float64)
    u, pu = _c(u, np.float64)
    assert g.shape == u.shape
    h = np.empty(g.shape, dtype=np.float64)
    _L().orc_swiglu(pg, pu, g.size, h.ctypes.data)
    return h


def rmsnorm(x_bits: np.ndarray, gain_bits: np.ndarray, eps: float) -> np.ndarray:
    """RMS-normalised rows of bf16 x [M][K] times the bf16 gain [K], fp64."""
    x, px = _c(np.atleast_2d(x_bits), np.uint16)
    g, pg = _c(gain_bits, np.uint16)
    M, K = x.shape
    assert g.shape == (K,)
    out = np.empty((M, K), dtype=np.float64)
    _L().orc_rmsnorm(px, pg, M, K, float(eps), out.ctypes.data)
    return out


def e8m0_value(code: int) -> float:
    return _L().orc_e8m0_value(int(code))


def mx_quantize(W_bits: np.ndarray):
    """MXFP4: bf16 W [N][K] (K % 32 == 0) -> (packed uint8 [N][K/2], E8M0 scales uint8 [N][K/32])."""
    W, pw = _c(W_bits, np.uint16)
    N, K = W.shape
    packed = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 32), dtype=np.uint8)
    if _L().orc_mx_quantize(pw, N, K, packed.ctypes.data, scales.ctypes.data) != 0:
        raise ValueError("mx_quantize: bad shape %r" % (W.shape,))
    return packed, scales


def mx_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    N, K = packed.shape[0], packed.shape[1] * 2
    out = np.empty((N, K), dtype=np.float64)
    _L().orc_mx_dequant(pp, ps, N, K, out.ctypes.data)
    return out


def mx_gemv(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray):
    """fp64 MXFP4 product (y [M][N], l1 [M][N]) for bf16 x [M][K]."""
    x, px = _c(np.atleast_2d(x_bits), np.uint16)
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    M, K = x.shape
    N = packed.shape[0]
    assert packed.shape[1] * 2 == K and scales.shape == (N, K // 32)
    y = np.empty((M, N), dtype=np.float64)
    l1 = np.empty((M, N), dtype=np.float64)
    _L().orc_mx_gemv(px, M, pp, ps, N, K, y.ctypes.data, l1.ctypes.data)
    return y, l1


def mx_a4_product(xq_packed: np.ndarray, xq_scales: np.ndarray, w_packed: np.ndarray, w_scales: np.ndarray):
    """fp64 product of two MXFP4 operands (y [M][N], l1 [M][N]): activation
    rows quantised by mx_quantize (the rows of x taken as the rows of a
    matrix) times MXFP4 weights, y = dequant(xq) @ dequant(w)^T and the error
    scale l1 = |dequant(xq)| @ |dequant(w)|^T, with fp64 sums (a library
    matrix product as the summation step). Page "github.com/kekzl/imp", the
    feature table: MXFP4 in the quantisation row and a block-scaled GEMM in
    the engine row; both operands block-scaled FP4 is the form that runs at
    the matrix cores' FP4 rate."""
    A = mx_dequant(xq_packed, xq_scales)
    B = mx_dequant(w_packed, w_scales)
    assert A.shape[1] == B.shape[1]
    return A @ B.T, np.abs(A) @ np.abs(B).T


def mx_tile(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Canonical MXFP4 -> the GPU library's MXFP4 tiled layout (4352-byte tiles)."""
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    N, K = packed.shape[0], packed.shape[1] * 2
    G, C = (N + 7) // 8, (K + 1023) // 1024
    t = np.empty(G * C * 4352, dtype=np.uint8)
    _L().orc_mx_tile(pp, ps, N, K, t.ctypes.data)
    return t


def tile(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Canonical -> the GPU library's tiled layout (one flat uint8 array of
    4608-byte tiles holding codes and scales)."""
    packed, pp = _c(packed, np.uint8)
    scales, ps = _c(scales, np.uint8)
    N, K = packed.shape[0], packed.shape[1] * 2
    G, C = (N + 7) // 8, (K + 1023) // 1024
    t = np.empty(G * C * 4608, dtype=np.uint8)
    _L().orc_tile(pp, ps, N, K, t.ctypes.data)
    return t


def tolerance_ok(y_gpu: np.ndarray, y_ref: np.ndarray, l1: np.ndarray, rel: float = 2e-3):
    """Per-element bound |y_gpu - y_ref| <= rel * l1; returns (ok, worst ratio)."""
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    bound = rel * l1
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return bool(np.all(err <= bound)), float(ratio.max() if ratio.size else 0.0)


def argmax_rows(y: np.ndarray) -> np.ndarray:
    """Greedy choice per row of y [M][N] (float32 or float64, decided in that
    precision): the first index of the largest value, a NaN ranking above
    every number, -0 equal to +0. Returns int32 [M]."""
    y = np.atleast_2d(y)
    if y.dtype == np.float32:
        y, py = _c(y, np.float32)
        f = _L().orc_argmax_rows_f32
    else:
        y, py = _c(y, np.float64)
        f = _L().orc_argmax_rows_f64
    M, N = y.shape
    if N < 1:
        raise ValueError("argmax_rows: empty rows")
    idx = np.empty(M, dtype=np.int32)
    f(py, M, N, N, idx.ctypes.data)
    return idx
