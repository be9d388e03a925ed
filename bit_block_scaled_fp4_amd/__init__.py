"""NVFP4 decode path for AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over libfp4.so, the C ABI declared in include/fp4.h.
It only marshals arguments: every step runs in the library's HIP kernels on
the tensors' device, on torch's current stream. PyTorch supplies device
memory and streams. There is no CPU fallback: without the built library the
import fails, and CPU tensors are rejected.

Names follow the C ABI: quantize, quantize_fp8, retile, gemv, gemv_multi, gemm_prefill,
gemm_prefill_multi, argmax_rows, lm_head_greedy, layout_bytes, workspace_bytes. The
products take an optional `workspace` (a zero-filled uint8 GPU tensor, see
new_workspace), which selects the C ABI's *_ws forms.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch  # loads the HIP runtime first; libfp4 then binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fp4.h")

ROWMAJOR, TILED, MX_ROWMAJOR, MX_TILED, MX_ACT = 0, 1, 2, 3, 4
MAX_PROJ = 8
OP_GEMV, OP_GEMM_PREFILL, OP_ARGMAX_ROWS, OP_LM_HEAD_GREEDY, OP_GEMV_RMSNORM, OP_GEMV_SWIGLU = 0, 1, 2, 3, 4, 5
_LAYOUTS = {"rowmajor": ROWMAJOR, "tiled": TILED, "mx_rowmajor": MX_ROWMAJOR, "mx_tiled": MX_TILED, "mx_act": MX_ACT,
            ROWMAJOR: ROWMAJOR, TILED: TILED, MX_ROWMAJOR: MX_ROWMAJOR, MX_TILED: MX_TILED, MX_ACT: MX_ACT}

if not os.path.exists(LIB_PATH):
    raise ImportError("libfp4.so is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python bit_block_scaled_fp4_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


class _Proj(ctypes.Structure):
    _fields_ = [("packed", _P), ("scales", _P), ("gscale", _P), ("N", _I64), ("y", _P), ("ldy", _I64)]


_lib.fp4_status_string.argtypes = [_I]
_lib.fp4_status_string.restype = ctypes.c_char_p
_lib.fp4_layout_bytes.argtypes = [_I64, _I64, _I, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
_lib.fp4_quantize.argtypes = [_P, _I64, _I64, _I, _P, _P, _P, _P]
_lib.fp4_quantize_fp8.argtypes = [_P, _P, _I64, _I64, _I, _P, _P, _P, _P]
_lib.fp4_retile.argtypes = [_P, _P, _I64, _I64, _P, _P, _P]
_SZ = ctypes.c_size_t
_lib.fp4_gemv.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]
_lib.fp4_gemv_ws.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
_lib.fp4_gemv_multi.argtypes = [ctypes.POINTER(_Proj), _I, _P, _I64, _I64, _P]
_lib.fp4_gemv_multi_ws.argtypes = [ctypes.POINTER(_Proj), _I, _P, _I64, _I64, _P, _SZ, _P]
_lib.fp4_gemm_prefill.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]
_lib.fp4_gemm_prefill_ws.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
_lib.fp4_gemm_prefill_multi.argtypes = [ctypes.POINTER(_Proj), _I, _P, _I64, _I64, _P]
_lib.fp4_gemm_prefill_multi_ws.argtypes = [ctypes.POINTER(_Proj), _I, _P, _I64, _I64, _P, _SZ, _P]
_lib.fp4_argmax_rows.argtypes = [_P, _P, _I64, _I64, _I64, _P, _SZ, _P]
_lib.fp4_lm_head_greedy.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
_lib.fp4_workspace_bytes.argtypes = [_I, _I64, _I64, ctypes.POINTER(_I64), _I, ctypes.POINTER(_SZ)]
_lib.fp4_quantize_mx.argtypes = [_P, _I64, _I64, _I, _P, _P, _P]
_lib.fp4_gemv_mx.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
_lib.fp4_gemm_prefill_mx.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
_lib.fp4_gemm_mx_a4.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P]
_lib.fp4_gemv_multi_rmsnorm.argtypes = [ctypes.POINTER(_Proj), _I, _P, _P, ctypes.c_float, _I64, _I64, _P, _SZ, _P]
_lib.fp4_gemv_swiglu.argtypes = [_P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
for _f in ("fp4_layout_bytes", "fp4_quantize", "fp4_quantize_fp8", "fp4_retile", "fp4_gemv", "fp4_gemv_ws",
           "fp4_gemv_multi", "fp4_gemv_multi_ws", "fp4_gemm_prefill", "fp4_gemm_prefill_ws", "fp4_gemm_prefill_multi",
           "fp4_gemm_prefill_multi_ws", "fp4_argmax_rows", "fp4_lm_head_greedy", "fp4_workspace_bytes",
           "fp4_gemv_multi_rmsnorm", "fp4_gemv_swiglu", "fp4_quantize_mx", "fp4_gemv_mx", "fp4_gemm_prefill_mx"):
    getattr(_lib, _f).restype = _I


class Fp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, _lib.fp4_status_string(status).decode(), status))


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Fp4Error(status, where)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s); there is no CPU path" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def layout_bytes(N: int, K: int, layout="tiled"):
    """(packed_bytes, scale_bytes) for an N x K weight in the given layout."""
    pb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.fp4_layout_bytes(N, K, _LAYOUTS[layout], ctypes.byref(pb), ctypes.byref(sb)), "fp4_layout_bytes")
    return pb.value, sb.value


def workspace_bytes(op: int, M: int, K: int, Ns: Sequence[int]) -> int:
    """fp4_workspace_bytes: workspace bytes a call of `op` (OP_GEMV,
    OP_GEMM_PREFILL, OP_ARGMAX_ROWS, OP_LM_HEAD_GREEDY) needs on the current
    device for M rows, K inputs and projections of Ns[i] outputs."""
    n = len(Ns)
    arr = (_I64 * max(1, n))(*Ns)
    out = ctypes.c_size_t()
    _check(_lib.fp4_workspace_bytes(int(op), M, K, arr, n, ctypes.byref(out)), "fp4_workspace_bytes")
    return out.value


def new_workspace(nbytes: int, device=None) -> torch.Tensor:
    """A zero-filled uint8 GPU tensor to pass as `workspace` (at least 1 byte;
    torch's allocator aligns it to 512 bytes). Allocate it once and reuse it
    for calls that run one after another."""
    return torch.zeros(max(1, int(nbytes)), dtype=torch.uint8, device=device or torch.device("cuda"))


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _dev(ws, "workspace", torch.uint8), ws.numel()


@dataclass
class NVFP4Weight:
    """Quantised weight on the device: packed codes, E4M3 block scales and the
    fp32 tensor scale. In the tiled layout `packed` holds codes and scales
    together and `scales` is None."""
    packed: torch.Tensor
    scales: Optional[torch.Tensor]
    gscale: torch.Tensor
    N: int
    K: int
    layout: int = TILED


def _opt(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    return None if t is None else _dev(t, name, torch.uint8)


def quantize(W: torch.Tensor, layout="tiled", out: Optional[NVFP4Weight] = None) -> NVFP4Weight:
    """fp4_quantize: bf16 W [N][K] -> NVFP4Weight in `layout`."""
    N, K = W.shape
    lay = _LAYOUTS[layout]
    if out is None:
        pb, sb = layout_bytes(N, K, lay)
        out = NVFP4Weight(torch.empty(pb, dtype=torch.uint8, device=W.device),
                          torch.empty(sb, dtype=torch.uint8, device=W.device) if lay == ROWMAJOR else None,
                          torch.empty(1, dtype=torch.float32, device=W.device), N, K, lay)
    _check(_lib.fp4_quantize(_dev(W, "W", torch.bfloat16), N, K, lay, _dev(out.packed, "packed", torch.uint8),
                             _opt(out.scales, "scales"), _dev(out.gscale, "gscale", torch.float32),
                             _stream(W.device)), "fp4_quantize")
    return out


@dataclass
class MXFP4Weight:
    """MXFP4 weight on the device: E2M1 codes and E8M0 scales per 32 elements
    (no tensor scale). In the MX tiled layout `packed` holds both and
    `scales` is None."""
    packed: torch.Tensor
    scales: Optional[torch.Tensor]
    N: int
    K: int
    layout: int = MX_TILED


def quantize_mx(W: torch.Tensor, layout="mx_tiled", out: Optional[MXFP4Weight] = None) -> MXFP4Weight:
    """fp4_quantize_mx: bf16 W [N][K] (K % 32 == 0; "mx_act" K % 128 == 0) ->
    MXFP4Weight in `layout` ("mx_act": the activation operand of gemm_mx_a4)."""
    N, K = W.shape
    lay = _LAYOUTS[layout]
    if lay not in (MX_ROWMAJOR, MX_TILED, MX_ACT):
        raise ValueError("quantize_mx takes an MX layout")
    if out is None:
        pb, sb = layout_bytes(N, K, lay)
        out = MXFP4Weight(torch.empty(pb, dtype=torch.uint8, device=W.device),
                          torch.empty(sb, dtype=torch.uint8, device=W.device) if lay != MX_TILED else None, N, K, lay)
    _check(_lib.fp4_quantize_mx(_dev(W, "W", torch.bfloat16), N, K, lay, _dev(out.packed, "packed", torch.uint8),
                                _opt(out.scales, "scales"), _stream(W.device)), "fp4_quantize_mx")
    return out


def _mx_tiled(w: MXFP4Weight) -> None:
    if w.layout != MX_TILED:
        raise ValueError("the MXFP4 products take MX tiled weights (quantize_mx(..., 'mx_tiled'))")


def gemv_mx(x: torch.Tensor, w: MXFP4Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_gemv_mx: y[M][N] = x @ dequant(w)^T (fp32) for an MXFP4 weight."""
    x, M, K = _x2d(x)
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    _mx_tiled(w)
    out = _out(out, (M, w.N), torch.float32, x.device, "out")
    _check(_lib.fp4_gemv_mx(_dev(out, "y", torch.float32), _dev(x, "x", torch.bfloat16), _dev(w.packed, "packed"),
                            M, w.N, K, _stream(x.device)), "fp4_gemv_mx")
    return out


def gemm_mx_a4(xq: MXFP4Weight, w: MXFP4Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_gemm_mx_a4: y[M][N] = dequant(xq) @ dequant(w)^T (fp32) with both
    operands MXFP4: xq the activation rows from quantize_mx(x, "mx_act"),
    w an MX tiled weight."""
    if xq.layout != MX_ACT or xq.scales is None:
        raise ValueError("xq must come from quantize_mx(x, 'mx_act')")
    if xq.K != w.K:
        raise ValueError("xq has K=%d, weight has K=%d" % (xq.K, w.K))
    _mx_tiled(w)
    out = _out(out, (xq.N, w.N), torch.float32, xq.packed.device, "out")
    _check(_lib.fp4_gemm_mx_a4(_dev(out, "y", torch.float32), _dev(xq.packed, "xq_packed", torch.uint8),
                               _dev(xq.scales, "xq_scales", torch.uint8), _dev(w.packed, "packed"), xq.N, w.N, w.K,
                               _stream(xq.packed.device)), "fp4_gemm_mx_a4")
    return out


def gemm_prefill_mx(x: torch.Tensor, w: MXFP4Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_gemm_prefill_mx: the MXFP4 product on bf16 MFMA for prefill-sized M."""
    x, M, K = _x2d(x)
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    _mx_tiled(w)
    out = _out(out, (M, w.N), torch.float32, x.device, "out")
    _check(_lib.fp4_gemm_prefill_mx(_dev(out, "y", torch.float32), _dev(x, "x", torch.bfloat16),
                                    _dev(w.packed, "packed"), M, w.N, K, _stream(x.device)), "fp4_gemm_prefill_mx")
    return out


def quantize_fp8(W: torch.Tensor, w_scale: torch.Tensor, layout="tiled",
                 out: Optional[NVFP4Weight] = None) -> NVFP4Weight:
    """fp4_quantize_fp8: FP8 E4M3 W [N][K] (torch.float8_e4m3fn or uint8 codes)
    with its fp32 dequantisation scale (a 1-element GPU tensor) -> NVFP4Weight."""
    N, K = W.shape
    if W.dtype == torch.float8_e4m3fn:
        W = W.view(torch.uint8)
    lay = _LAYOUTS[layout]
    if out is None:
        pb, sb = layout_bytes(N, K, lay)
        out = NVFP4Weight(torch.empty(pb, dtype=torch.uint8, device=W.device),
                          torch.empty(sb, dtype=torch.uint8, device=W.device) if lay == ROWMAJOR else None,
                          torch.empty(1, dtype=torch.float32, device=W.device), N, K, lay)
    _check(_lib.fp4_quantize_fp8(_dev(W, "W", torch.uint8), _dev(w_scale, "w_scale", torch.float32), N, K, lay,
                                 _dev(out.packed, "packed", torch.uint8), _opt(out.scales, "scales"),
                                 _dev(out.gscale, "gscale", torch.float32), _stream(W.device)), "fp4_quantize_fp8")
    return out


def retile(w: NVFP4Weight, out: Optional[NVFP4Weight] = None) -> NVFP4Weight:
    """fp4_retile: canonical (row-major) NVFP4Weight -> tiled copy (gscale shared)."""
    if w.layout != ROWMAJOR:
        raise ValueError("retile expects a row-major weight")
    if out is None:
        pb, _ = layout_bytes(w.N, w.K, TILED)
        out = NVFP4Weight(torch.empty(pb, dtype=torch.uint8, device=w.packed.device), None, w.gscale, w.N, w.K, TILED)
    _check(_lib.fp4_retile(_dev(w.packed, "packed", torch.uint8), _dev(w.scales, "scales", torch.uint8), w.N, w.K,
                           _dev(out.packed, "packed_tiled", torch.uint8), None, _stream(w.packed.device)),
           "fp4_retile")
    return out


def _tiled(w: NVFP4Weight) -> None:
    if w.layout != TILED:
        raise ValueError("the products take tiled weights (quantize(..., 'tiled') or retile())")


def _x2d(x: torch.Tensor):
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dim() != 2:
        raise ValueError("x must be [K] or [M][K]")
    return x, x.shape[0], x.shape[1]


def _out(out: Optional[torch.Tensor], shape, dtype, device, name: str) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(out.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(out.shape)))
    return out


def gemv(x: torch.Tensor, w: NVFP4Weight, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_gemv (fp4_gemv_ws with a workspace): y[M][N] = x[M][K] @ dequant(w)^T
    (fp32), x bf16, w tiled."""
    x, M, K = _x2d(x)
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    out = _out(out, (M, w.N), torch.float32, x.device, "out")
    _tiled(w)
    args = (_dev(out, "y", torch.float32), _dev(x, "x", torch.bfloat16), _dev(w.packed, "packed"), None,
            _dev(w.gscale, "gscale", torch.float32), M, w.N, K)
    if workspace is None:
        _check(_lib.fp4_gemv(*args, _stream(x.device)), "fp4_gemv")
    else:
        _check(_lib.fp4_gemv_ws(*args, *_ws(workspace), _stream(x.device)), "fp4_gemv_ws")
    return out


def _projs(M: int, K: int, weights: Sequence[NVFP4Weight], outs: Sequence[torch.Tensor],
           ldys: Optional[Sequence[int]]):
    """The fp4_proj array of a fused launch, after checking every output's extent."""
    n = len(weights)
    if not 1 <= n <= MAX_PROJ or len(outs) != n:
        raise ValueError("need 1..%d weights and as many outputs" % MAX_PROJ)
    arr = (_Proj * n)()
    for i, (w, y) in enumerate(zip(weights, outs)):
        if w.K != K:
            raise ValueError("weight %d has K=%d, x has K=%d" % (i, w.K, K))
        ldy = ldys[i] if ldys is not None else w.N
        if y.device.type != "cuda" or y.dtype != torch.float32:
            raise ValueError("outs[%d] must be a float32 GPU tensor" % i)
        avail = y.untyped_storage().nbytes() // 4 - y.storage_offset()   # fp32 elements from y's data_ptr on
        if avail < (M - 1) * ldy + w.N:
            raise ValueError("outs[%d] is too small for M=%d rows of stride %d" % (i, M, ldy))
        _tiled(w)
        arr[i] = _Proj(_dev(w.packed, "packed"), None, _dev(w.gscale, "gscale", torch.float32), w.N, y.data_ptr(), ldy)
    return arr, n


def gemv_multi(x: torch.Tensor, weights: Sequence[NVFP4Weight], outs: Sequence[torch.Tensor],
               ldys: Optional[Sequence[int]] = None, workspace: Optional[torch.Tensor] = None) -> None:
    """fp4_gemv_multi (fp4_gemv_multi_ws with a workspace): one launch computing
    outs[i][m][n] (row stride ldys[i]) for every weight."""
    x, M, K = _x2d(x)
    arr, n = _projs(M, K, weights, outs, ldys)
    if workspace is None:
        _check(_lib.fp4_gemv_multi(arr, n, _dev(x, "x", torch.bfloat16), M, K, _stream(x.device)), "fp4_gemv_multi")
    else:
        _check(_lib.fp4_gemv_multi_ws(arr, n, _dev(x, "x", torch.bfloat16), M, K, *_ws(workspace), _stream(x.device)),
               "fp4_gemv_multi_ws")


def gemv_multi_rmsnorm(x: torch.Tensor, gain: torch.Tensor, eps: float, weights: Sequence[NVFP4Weight],
                       outs: Sequence[torch.Tensor], ldys: Optional[Sequence[int]] = None,
                       workspace: Optional[torch.Tensor] = None) -> None:
    """fp4_gemv_multi_rmsnorm: outs[i] = RMSNorm(x; gain, eps) @ dequant(weights[i])^T
    (gain bf16 [K]); needs a workspace beyond 2 rows (workspace_bytes(OP_GEMV_RMSNORM, ...))."""
    x, M, K = _x2d(x)
    if gain.numel() != K:
        raise ValueError("gain must have K=%d elements" % K)
    arr, n = _projs(M, K, weights, outs, ldys)
    _check(_lib.fp4_gemv_multi_rmsnorm(arr, n, _dev(x, "x", torch.bfloat16), _dev(gain, "gain", torch.bfloat16),
                                       float(eps), M, K, *_ws(workspace), _stream(x.device)), "fp4_gemv_multi_rmsnorm")


def gemv_swiglu(x: torch.Tensor, gate: NVFP4Weight, up: NVFP4Weight, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_gemv_swiglu: h = bf16(silu(x @ dequant(gate)^T) * (x @ dequant(up)^T)), bf16 [M][N]."""
    x, M, K = _x2d(x)
    if gate.K != K or up.K != K or gate.N != up.N:
        raise ValueError("gate and up must be [N][K] with the K of x")
    _tiled(gate)
    _tiled(up)
    out = _out(out, (M, gate.N), torch.bfloat16, x.device, "out")
    _check(_lib.fp4_gemv_swiglu(_dev(out, "h", torch.bfloat16), gate.N, _dev(x, "x", torch.bfloat16),
                                _dev(gate.packed, "gate"), _dev(gate.gscale, "gate gscale", torch.float32),
                                _dev(up.packed, "up"), _dev(up.gscale, "up gscale", torch.float32), M, gate.N, K,
                                *_ws(workspace), _stream(x.device)), "fp4_gemv_swiglu")
    return out


def gemm_prefill_multi(x: torch.Tensor, weights: Sequence[NVFP4Weight], outs: Sequence[torch.Tensor],
                       ldys: Optional[Sequence[int]] = None, workspace: Optional[torch.Tensor] = None) -> None:
    """fp4_gemm_prefill_multi (fp4_gemm_prefill_multi_ws with a workspace): one
    matrix-core launch computing outs[i][m][n] (row stride ldys[i]) for every weight."""
    x, M, K = _x2d(x)
    arr, n = _projs(M, K, weights, outs, ldys)
    if workspace is None:
        _check(_lib.fp4_gemm_prefill_multi(arr, n, _dev(x, "x", torch.bfloat16), M, K, _stream(x.device)),
               "fp4_gemm_prefill_multi")
    else:
        _check(_lib.fp4_gemm_prefill_multi_ws(arr, n, _dev(x, "x", torch.bfloat16), M, K, *_ws(workspace),
                                              _stream(x.device)), "fp4_gemm_prefill_multi_ws")


def gemm_prefill(x: torch.Tensor, w: NVFP4Weight, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_gemm_prefill (fp4_gemm_prefill_ws with a workspace): the same product
    on bf16 MFMA for prefill-sized M."""
    x, M, K = _x2d(x)
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    out = _out(out, (M, w.N), torch.float32, x.device, "out")
    _tiled(w)
    args = (_dev(out, "y", torch.float32), _dev(x, "x", torch.bfloat16), _dev(w.packed, "packed"), None,
            _dev(w.gscale, "gscale", torch.float32), M, w.N, K)
    if workspace is None:
        _check(_lib.fp4_gemm_prefill(*args, _stream(x.device)), "fp4_gemm_prefill")
    else:
        _check(_lib.fp4_gemm_prefill_ws(*args, *_ws(workspace), _stream(x.device)), "fp4_gemm_prefill_ws")
    return out


def argmax_rows(y: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4_argmax_rows: int32 [M], per row of fp32 y [M][N] (or [N]) the first
    index of the largest value (NaN above every number, -0 equal to +0)."""
    y2 = y.view(1, -1) if y.dim() == 1 else y
    if y2.dim() != 2:
        raise ValueError("y must be [N] or [M][N]")
    M, N = y2.shape
    out = _out(out, (M,), torch.int32, y.device, "out")
    _check(_lib.fp4_argmax_rows(_dev(out, "idx", torch.int32), _dev(y2, "y", torch.float32), M, N, N,
                                *_ws(workspace), _stream(y.device)), "fp4_argmax_rows")
    return out


def lm_head_greedy(x: torch.Tensor, w: NVFP4Weight, logits: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """fp4_lm_head_greedy: (idx int32 [M], logits fp32 [M][N]) with logits =
    x @ dequant(w)^T and idx the greedy choice of each row."""
    x, M, K = _x2d(x)
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    logits = _out(logits, (M, w.N), torch.float32, x.device, "logits")
    out = _out(out, (M,), torch.int32, x.device, "out")
    _tiled(w)
    _check(_lib.fp4_lm_head_greedy(_dev(out, "idx", torch.int32), _dev(logits, "logits", torch.float32),
                                   _dev(x, "x", torch.bfloat16), _dev(w.packed, "packed"), None,
                                   _dev(w.gscale, "gscale", torch.float32), M, w.N, K, *_ws(workspace),
                                   _stream(x.device)), "fp4_lm_head_greedy")
    return out, logits


def raw():
    """The ctypes handle of libfp4.so (for tests that call the C ABI directly)."""
    return _lib


__all__ = ["quantize", "quantize_fp8", "retile", "gemv", "gemv_multi", "gemm_prefill", "gemm_prefill_multi",
           "argmax_rows", "lm_head_greedy", "gemv_multi_rmsnorm", "gemv_swiglu", "layout_bytes", "workspace_bytes",
           "new_workspace", "NVFP4Weight", "OP_GEMV", "OP_GEMM_PREFILL", "OP_ARGMAX_ROWS", "OP_LM_HEAD_GREEDY",
           "OP_GEMV_RMSNORM", "OP_GEMV_SWIGLU", "MXFP4Weight", "quantize_mx", "gemv_mx", "gemm_prefill_mx", "gemm_mx_a4",
           "Fp4Error", "raw", "ROWMAJOR", "TILED", "LIB_PATH", "HEADER_PATH"]
