"""The C-ABI library loads, exports every function include/fp4.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed:
none of these calls reaches a launch)."""
import ctypes
import re

import pytest

import bit_block_scaled_fp4_amd as fp4

OK, ENULL, ESHAPE, EALIGN, ELAYOUT, EWS = 0, -1, -2, -3, -4, -7
A = 1 << 20          # a fake, 16-byte-aligned address; never dereferenced


def declared_functions(path=None):
    src = open(path or fp4.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|void|size_t|const char)\s*\*?\s*(fp4_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names == sorted(["fp4_status_string", "fp4_layout_bytes", "fp4_quantize", "fp4_retile", "fp4_gemv",
                            "fp4_gemv_ws", "fp4_gemv_multi", "fp4_gemv_multi_ws", "fp4_gemm_prefill",
                            "fp4_gemm_prefill_ws", "fp4_gemm_prefill_multi", "fp4_gemm_prefill_multi_ws",
                            "fp4_argmax_rows", "fp4_lm_head_greedy", "fp4_quantize_fp8", "fp4_workspace_bytes",
                            "fp4_gemv_multi_noalloc", "fp4_gemv_multi_rmsnorm", "fp4_gemv_swiglu",
                            "fp4_quantize_mx", "fp4_gemv_mx", "fp4_gemm_prefill_mx", "fp4_gemm_mx_a4"])
    lib = ctypes.CDLL(fp4.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    import os
    for h in sorted(os.listdir(os.path.dirname(fp4.HEADER_PATH))):   # every header under include/
        for n in declared_functions(os.path.join(os.path.dirname(fp4.HEADER_PATH), h)):
            assert hasattr(lib, n), (h, n)


def test_status_strings():
    lib = fp4.raw()
    for s in (OK, ENULL, ESHAPE, EALIGN, ELAYOUT, -5, -6, -7, 42):
        assert isinstance(lib.fp4_status_string(s), bytes) and lib.fp4_status_string(s)


def test_layout_bytes():
    assert fp4.layout_bytes(1024, 1024, "rowmajor") == (1024 * 512, 1024 * 64)
    # tiled: 4608-byte tiles of codes and scales together, no separate scale array
    assert fp4.layout_bytes(1024, 1024, "tiled") == (128 * 4608, 0)
    assert fp4.layout_bytes(11, 1040, "tiled") == (2 * 2 * 4608, 0)
    assert fp4.layout_bytes(151936, 1024, "tiled") == (151936 * 576, 0)
    with pytest.raises(fp4.Fp4Error) as e:
        fp4.layout_bytes(8, 24)
    assert e.value.status == ESHAPE
    with pytest.raises(KeyError):
        fp4.layout_bytes(8, 32, "columnmajor")
    pb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert fp4.raw().fp4_layout_bytes(8, 32, 7, ctypes.byref(pb), ctypes.byref(sb)) == ELAYOUT
    assert fp4.raw().fp4_layout_bytes(8, 32, 0, None, ctypes.byref(sb)) == ENULL


def test_gemv_argument_errors():
    L = fp4.raw()
    assert L.fp4_gemv(None, A, A, A, A, 1, 8, 32, None) == ENULL
    assert L.fp4_gemv(A, A, A, A, None, 1, 8, 32, None) == ENULL
    assert L.fp4_gemv(A, A, A, A, A, 0, 8, 32, None) == ESHAPE
    assert L.fp4_gemv(A, A, A, A, A, 1, 0, 32, None) == ESHAPE
    assert L.fp4_gemv(A, A, A, A, A, 1, 8, 24, None) == ESHAPE
    assert L.fp4_gemv(A, A, A, A, A, 1, 8, 0, None) == ESHAPE
    assert L.fp4_gemv(A, A, A, A, A, 1, 1 << 29, 32, None) == ESHAPE
    assert L.fp4_gemv(A, A + 8, A, A, A, 1, 8, 32, None) == EALIGN
    assert L.fp4_gemv(A, A, A + 4, A, A, 1, 8, 32, None) == EALIGN
    assert L.fp4_gemv(A + 2, A, A, A, A, 1, 8, 32, None) == EALIGN


def test_gemv_multi_argument_errors():
    L = fp4.raw()
    P = (fp4._Proj * 9)()
    for i in range(9):
        P[i] = fp4._Proj(A, A, A, 8, A, 8)
    assert L.fp4_gemv_multi(None, 1, A, 1, 32, None) == ENULL
    assert L.fp4_gemv_multi(P, 0, A, 1, 32, None) == ESHAPE
    assert L.fp4_gemv_multi(P, 9, A, 1, 32, None) == ESHAPE
    P[1] = fp4._Proj(A, A, A, 8, A, 4)                 # ldy < N
    assert L.fp4_gemv_multi(P, 2, A, 1, 32, None) == ESHAPE
    P[1] = fp4._Proj(None, A, A, 8, A, 8)
    assert L.fp4_gemv_multi(P, 2, A, 1, 32, None) == ENULL
    P[1] = fp4._Proj(A + 1, A, A, 8, A, 8)
    assert L.fp4_gemv_multi(P, 2, A, 1, 32, None) == EALIGN


def test_quantize_retile_prefill_argument_errors():
    L = fp4.raw()
    assert L.fp4_quantize(None, 8, 32, 1, A, A, A, None) == ENULL
    assert L.fp4_quantize(A, 8, 32, 0, A, None, A, None) == ENULL    # row-major needs the scale array
    assert L.fp4_quantize(A, 8, 30, 1, A, A, A, None) == ESHAPE
    assert L.fp4_quantize(A, 8, 32, 3, A, A, A, None) == ELAYOUT
    assert L.fp4_quantize(A + 8, 8, 32, 1, A, A, A, None) == EALIGN
    assert L.fp4_retile(A, A, 8, 32, None, A, None) == ENULL
    assert L.fp4_retile(A, A, -1, 32, A, A, None) == ESHAPE
    assert L.fp4_retile(A + 4, A, 8, 32, A, A, None) == EALIGN
    assert L.fp4_gemm_prefill(A, A, A, A, None, 4, 8, 32, None) == ENULL
    assert L.fp4_gemm_prefill(A, A, A, A, A, 0, 8, 32, None) == ESHAPE
    assert L.fp4_gemm_prefill(A, A + 2, A, A, A, 4, 8, 32, None) == EALIGN
    # 256-row slabs of x (256*K*2 bytes) or y (256*N*4 bytes) reaching 2 GB
    assert L.fp4_gemm_prefill(A, A, A, A, A, 4, 8, 1 << 22, None) == ESHAPE
    assert L.fp4_gemm_prefill(A, A, A, A, A, 4, 1 << 21, 32, None) == ESHAPE


def test_gemm_prefill_multi_argument_errors():
    L = fp4.raw()
    P = (fp4._Proj * 9)()
    for i in range(9):
        P[i] = fp4._Proj(A, A, A, 8, A, 8)
    assert L.fp4_gemm_prefill_multi(None, 1, A, 4, 32, None) == ENULL
    assert L.fp4_gemm_prefill_multi(P, 1, None, 4, 32, None) == ENULL
    assert L.fp4_gemm_prefill_multi(P, 0, A, 4, 32, None) == ESHAPE
    assert L.fp4_gemm_prefill_multi(P, 9, A, 4, 32, None) == ESHAPE
    assert L.fp4_gemm_prefill_multi(P, 2, A, 0, 32, None) == ESHAPE
    assert L.fp4_gemm_prefill_multi(P, 2, A, 4, 24, None) == ESHAPE
    assert L.fp4_gemm_prefill_multi(P, 2, A + 2, 4, 32, None) == EALIGN
    assert L.fp4_gemm_prefill_multi(P, 2, A, 4, 1 << 22, None) == ESHAPE        # x slab of 2 GB
    P[1] = fp4._Proj(A, A, A, 8, A, 4)                                          # ldy < N
    assert L.fp4_gemm_prefill_multi(P, 2, A, 4, 32, None) == ESHAPE
    P[1] = fp4._Proj(A, A, A, 8, A, 1 << 21)                                    # y slab of 2 GB
    assert L.fp4_gemm_prefill_multi(P, 2, A, 4, 32, None) == ESHAPE
    P[1] = fp4._Proj(A, A, None, 8, A, 8)
    assert L.fp4_gemm_prefill_multi(P, 2, A, 4, 32, None) == ENULL
    P[1] = fp4._Proj(A, A, A, 8, A + 2, 8)
    assert L.fp4_gemm_prefill_multi(P, 2, A, 4, 32, None) == EALIGN


def test_argmax_and_greedy_argument_errors():
    L = fp4.raw()
    assert L.fp4_argmax_rows(None, A, 1, 8, 8, None, 0, None) == ENULL
    assert L.fp4_argmax_rows(A, None, 1, 8, 8, None, 0, None) == ENULL
    assert L.fp4_argmax_rows(A, A, 0, 8, 8, None, 0, None) == ESHAPE
    assert L.fp4_argmax_rows(A, A, 1, 0, 8, None, 0, None) == ESHAPE
    assert L.fp4_argmax_rows(A, A, 2, 8, 7, None, 0, None) == ESHAPE          # row stride below N
    assert L.fp4_argmax_rows(A, A, 1, 1 << 29, 1 << 29, None, 0, None) == ESHAPE
    assert L.fp4_argmax_rows(A + 2, A, 1, 8, 8, None, 0, None) == EALIGN
    assert L.fp4_argmax_rows(A, A + 1, 1, 8, 8, None, 0, None) == EALIGN
    # a workspace: 256-byte aligned, at least what fp4_workspace_bytes reports
    need = fp4.workspace_bytes(fp4.OP_ARGMAX_ROWS, 2, 0, [10000])
    assert need > 65536
    assert L.fp4_argmax_rows(A, A, 2, 10000, 10000, A + 16, need, None) == EALIGN
    assert L.fp4_argmax_rows(A, A, 2, 10000, 10000, A, need - 1, None) == EWS
    # the greedy step checks everything before its first launch
    assert L.fp4_lm_head_greedy(None, A, A, A, None, A, 1, 8, 32, None, 0, None) == ENULL
    assert L.fp4_lm_head_greedy(A, None, A, A, None, A, 1, 8, 32, None, 0, None) == ENULL
    assert L.fp4_lm_head_greedy(A, A, A, A, None, A, 1, 8, 24, None, 0, None) == ESHAPE
    assert L.fp4_lm_head_greedy(A, A, A, A, None, A, 0, 8, 32, None, 0, None) == ESHAPE
    assert L.fp4_lm_head_greedy(A + 2, A, A, A, None, A, 1, 8, 32, None, 0, None) == EALIGN
    assert L.fp4_lm_head_greedy(A, A, A + 8, A, None, A, 1, 8, 32, None, 0, None) == EALIGN
    need = fp4.workspace_bytes(fp4.OP_LM_HEAD_GREEDY, 1, 1024, [151936])
    assert L.fp4_lm_head_greedy(A, A, A, A, None, A, 1, 151936, 1024, A, need - 8, None) == EWS


def test_workspace_bytes_query():
    """Sizes of the caller-owned workspaces: nothing for calls without
    scratch, the 64 KiB counter header plus the partial sums or keys
    otherwise; bad queries are rejected."""
    H = 65536
    assert fp4.workspace_bytes(fp4.OP_GEMV, 1, 17408, [5120]) == 0             # M = 1: vector ALUs, no split
    assert fp4.workspace_bytes(fp4.OP_GEMV, 8, 1024, [151936]) == 0            # one K chunk: no partials
    # M = 8 on 17 chunks: C * pairs * 16 * 16 fp32 partial sums
    assert fp4.workspace_bytes(fp4.OP_GEMV, 8, 17408, [5120]) == H + 17 * 320 * 1024
    assert fp4.workspace_bytes(fp4.OP_GEMV, 8, 5120, [17408, 17408]) == H + 5 * 2176 * 1024
    assert fp4.workspace_bytes(fp4.OP_ARGMAX_ROWS, 3, 0, [4096]) == 0          # one segment per row
    assert fp4.workspace_bytes(fp4.OP_ARGMAX_ROWS, 3, 0, [4097]) == H + 3 * 2 * 8
    assert fp4.workspace_bytes(fp4.OP_ARGMAX_ROWS, 600, 0, [8192]) == H + 512 * 2 * 8   # 512 rows per launch
    assert fp4.workspace_bytes(fp4.OP_LM_HEAD_GREEDY, 1, 1024, [151936]) == H     # keys in the header
    for bad in ((fp4.OP_GEMV, 0, 32, [8]), (fp4.OP_GEMV, 1, 24, [8]), (fp4.OP_ARGMAX_ROWS, 1, 0, [8, 8]),
                (fp4.OP_LM_HEAD_GREEDY, 1, 32, [0])):
        with pytest.raises(fp4.Fp4Error) as e:
            fp4.workspace_bytes(*bad)
        assert e.value.status == ESHAPE, bad
    with pytest.raises(fp4.Fp4Error) as e:
        fp4.workspace_bytes(9, 1, 32, [8])
    assert e.value.status == -6
    out = ctypes.c_size_t()
    assert fp4.raw().fp4_workspace_bytes(0, 1, 32, None, 1, ctypes.byref(out)) == ENULL


def test_quantize_fp8_argument_errors():
    L = fp4.raw()
    B = A + 4096         # another fake address (the tensor scale must not alias gscale)
    assert L.fp4_quantize_fp8(None, A, 8, 32, 1, A, None, B, None) == ENULL
    assert L.fp4_quantize_fp8(A, None, 8, 32, 1, A, None, B, None) == ENULL
    assert L.fp4_quantize_fp8(A, A, 8, 32, 0, A, None, B, None) == ENULL   # row-major needs the scale array
    assert L.fp4_quantize_fp8(A, A, 8, 30, 1, A, None, B, None) == ESHAPE
    assert L.fp4_quantize_fp8(A, A, 8, 32, 2, A, None, B, None) == ELAYOUT
    assert L.fp4_quantize_fp8(A + 8, A, 8, 32, 1, A, None, B, None) == EALIGN
    assert L.fp4_quantize_fp8(A, A + 2, 8, 32, 1, A, None, B, None) == EALIGN
    assert L.fp4_quantize_fp8(A, B, 8, 32, 1, A, None, B, None) == -6      # w_scale is gscale


def test_binding_rejects_cpu_tensors():
    import torch
    W = torch.zeros(8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fp4.quantize(W, out=fp4.NVFP4Weight(torch.zeros(1, dtype=torch.uint8), torch.zeros(1, dtype=torch.uint8),
                                            torch.zeros(1), 8, 32))
    with pytest.raises(ValueError, match="GPU tensor"):
        fp4.argmax_rows(torch.zeros(4, 8))


def test_binding_checks_fused_calls_before_any_gpu_work():
    """gemv_multi and gemm_prefill_multi reject mismatched K, a wrong number
    of outputs and more than FP4_MAX_PROJ projections in the binding, before
    any HIP call (CPU tensors suffice to reach these checks)."""
    import torch
    w = fp4.NVFP4Weight(torch.zeros(1, dtype=torch.uint8), None, torch.zeros(1), 8, 32)
    w64 = fp4.NVFP4Weight(torch.zeros(1, dtype=torch.uint8), None, torch.zeros(1), 8, 64)
    x = torch.zeros(2, 32, dtype=torch.bfloat16)
    y = torch.zeros(2, 8)
    for call in (fp4.gemv_multi, fp4.gemm_prefill_multi):
        with pytest.raises(ValueError, match="has K=64"):
            call(x, [w64, w], [y, y])
        with pytest.raises(ValueError, match="as many outputs"):
            call(x, [w, w], [y])
        with pytest.raises(ValueError, match="as many outputs"):
            call(x, [w] * (fp4.MAX_PROJ + 1), [y] * (fp4.MAX_PROJ + 1))
        with pytest.raises(ValueError, match="GPU tensor"):
            call(x, [w], [y])
    with pytest.raises(ValueError, match=r"\[K\] or \[M\]\[K\]"):
        fp4.gemm_prefill_multi(torch.zeros(2, 2, 32, dtype=torch.bfloat16), [w], [y])


def test_rmsnorm_and_swiglu_argument_errors():
    L = fp4.raw()
    P = (fp4._Proj * 1)(fp4._Proj(A, None, A, 8, A, 8))
    assert L.fp4_gemv_multi_rmsnorm(P, 1, A, None, 1e-6, 1, 32, None, 0, None) == ENULL
    assert L.fp4_gemv_multi_rmsnorm(P, 1, A, A + 2, 1e-6, 1, 32, None, 0, None) == EALIGN
    assert L.fp4_gemv_multi_rmsnorm(P, 1, A, A, -1.0, 1, 32, None, 0, None) == ESHAPE
    assert L.fp4_gemv_multi_rmsnorm(P, 1, A, A, float("nan"), 1, 32, None, 0, None) == ESHAPE
    assert L.fp4_gemv_multi_rmsnorm(P, 1, A, A, 1e-6, 1, 24, None, 0, None) == ESHAPE
    # 8 rows: the normalised rows go through the workspace, which is then required
    assert fp4.workspace_bytes(fp4.OP_GEMV_RMSNORM, 8, 1024, [8]) >= 65536 + 8 * 1024 * 2
    assert fp4.workspace_bytes(fp4.OP_GEMV_RMSNORM, 1, 1024, [8]) == 0
    assert L.fp4_gemv_multi_rmsnorm(P, 1, A, A, 1e-6, 8, 1024, None, 0, None) == EWS
    assert L.fp4_gemv_swiglu(None, 8, A, A, A, A, A, 1, 8, 32, None, 0, None) == ENULL
    assert L.fp4_gemv_swiglu(A, 8, A, A, None, A, A, 1, 8, 32, None, 0, None) == ENULL
    assert L.fp4_gemv_swiglu(A, 7, A, A, A, A, A, 1, 8, 32, None, 0, None) == ESHAPE     # ldh < N
    assert L.fp4_gemv_swiglu(A + 1, 8, A, A, A, A, A, 1, 8, 32, None, 0, None) == EALIGN
    assert L.fp4_gemv_swiglu(A, 8, A, A, A, A, A, 1, 8, 24, None, 0, None) == ESHAPE
    assert fp4.workspace_bytes(fp4.OP_GEMV_SWIGLU, 1, 5120, [17408]) == 0
    need = fp4.workspace_bytes(fp4.OP_GEMV_SWIGLU, 8, 5120, [17408])
    assert need >= 65536 + 2 * 8 * 17408 * 4
    assert L.fp4_gemv_swiglu(A, 17408, A, A, A, A, A, 8, 17408, 5120, None, 0, None) == EWS


def test_mx_layout_bytes_and_argument_errors():
    assert fp4.layout_bytes(1024, 1024, "mx_rowmajor") == (1024 * 512, 1024 * 32)
    assert fp4.layout_bytes(1024, 1024, "mx_tiled") == (128 * 4352, 0)
    assert fp4.layout_bytes(11, 1056, "mx_tiled") == (2 * 2 * 4352, 0)
    assert fp4.layout_bytes(1024, 1024, "mx_act") == (1024 * 512, 1024 * 32)
    with pytest.raises(fp4.Fp4Error) as e:
        fp4.layout_bytes(8, 96, "mx_act")                        # K % 128 != 0
    assert e.value.status == ESHAPE
    with pytest.raises(fp4.Fp4Error) as e:
        fp4.layout_bytes(8, 48, "mx_tiled")                      # K % 32 != 0
    assert e.value.status == ESHAPE
    L = fp4.raw()
    assert L.fp4_quantize_mx(A, 8, 64, 1, A, A, None) == ELAYOUT     # an NVFP4 layout
    assert L.fp4_quantize_mx(None, 8, 64, 3, A, None, None) == ENULL
    assert L.fp4_quantize_mx(A, 8, 64, 2, A, None, None) == ENULL     # row-major needs the scale array
    assert L.fp4_quantize_mx(A, 8, 128, 4, A, None, None) == ENULL    # so does the activation layout
    assert L.fp4_quantize_mx(A, 8, 96, 4, A, A, None) == ESHAPE       # activation layout: K % 128
    assert L.fp4_quantize_mx(A, 8, 128, 5, A, A, None) == ELAYOUT
    assert L.fp4_quantize_mx(A, 8, 48, 3, A, None, None) == ESHAPE
    assert L.fp4_quantize_mx(A + 8, 8, 64, 3, A, None, None) == EALIGN
    assert L.fp4_gemv_mx(None, A, A, 1, 8, 64, None) == ENULL
    assert L.fp4_gemv_mx(A, A, A, 1, 8, 48, None) == ESHAPE
    assert L.fp4_gemv_mx(A, A, A, 0, 8, 64, None) == ESHAPE
    assert L.fp4_gemv_mx(A, A + 8, A, 1, 8, 64, None) == EALIGN
    assert L.fp4_gemm_prefill_mx(A, A, None, 4, 8, 64, None) == ENULL
    assert L.fp4_gemm_prefill_mx(A, A, A, 4, 8, 1 << 22, None) == ESHAPE
    # both operands MXFP4: K % 128, the row limit of the grid, alignment
    L.fp4_gemm_mx_a4.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    assert L.fp4_gemm_mx_a4(A, A, None, A, 4, 8, 128, None) == ENULL
    assert L.fp4_gemm_mx_a4(None, A, A, A, 4, 8, 128, None) == ENULL
    assert L.fp4_gemm_mx_a4(A, A, A, A, 4, 8, 96, None) == ESHAPE        # K % 128 != 0
    assert L.fp4_gemm_mx_a4(A, A, A, A, 0, 8, 128, None) == ESHAPE
    assert L.fp4_gemm_mx_a4(A, A, A, A, 65535 * 256 + 1, 8, 128, None) == ESHAPE
    assert L.fp4_gemm_mx_a4(A, A, A, A, 1 << 20, 8, 1 << 16, None) == ESHAPE   # M*K/32 reaches 2^31
    assert L.fp4_gemm_mx_a4(A, A + 8, A, A, 4, 8, 128, None) == EALIGN   # codes not 16-byte aligned
    assert L.fp4_gemm_mx_a4(A, A, A + 2, A, 4, 8, 128, None) == EALIGN   # scales not 4-byte aligned
