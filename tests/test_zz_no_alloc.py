"""fp4_gemv_multi_noalloc (the product with its scratch in the library's fixed
device array, for callers that cannot allocate) against fp4_gemv_multi_ws (the
same kernels with a caller's workspace): equal outputs bit for bit on two calls
in a row, the second with a smaller input, both within the oracle's tolerance;
a call needing more scratch than the array holds is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_tensor

pytestmark = pytest.mark.gpu


def _gpu_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_noalloc_equals_workspace_form_on_two_calls():
    import bit_block_scaled_fp4_amd as fp4
    L = fp4.raw()
    L.fp4_gemv_multi_noalloc.argtypes = [ctypes.POINTER(fp4._Proj), ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p]
    L.fp4_gemv_multi_noalloc.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream
    # matrix-core path with K chunks (scratch in use), then a smaller call
    for M, K, Ns, seed in ((9, 3008, (333, 1000, 16), 1), (5, 2048, (200, 40), 2)):
        print("noalloc case", M, K, Ns, flush=True)
        bws = [bf16_tensor((N, K), 1300 + seed * 10 + i, 0.02, outlier_p=0.002, outlier_scale=20.0)
               for i, N in enumerate(Ns)]
        ws = [fp4.quantize(_gpu_bf16(b), "tiled") for b in bws]
        bx = bf16_tensor((M, K), 1400 + seed, 1.0)
        x = _gpu_bf16(bx)
        need = fp4.workspace_bytes(fp4.OP_GEMV, M, K, list(Ns))
        assert 65536 < need <= 16 << 20
        work = fp4.new_workspace(need)
        y_ws = [torch.full((M, N), float("nan"), device="cuda") for N in Ns]
        y_na = [torch.full((M, N), float("nan"), device="cuda") for N in Ns]
        a_ws, n = fp4._projs(M, K, ws, y_ws, None)
        a_na, _ = fp4._projs(M, K, ws, y_na, None)
        assert L.fp4_gemv_multi_ws(a_ws, n, x.data_ptr(), M, K, work.data_ptr(), work.numel(), stream) == 0
        assert L.fp4_gemv_multi_noalloc(a_na, n, x.data_ptr(), M, K, stream) == 0
        torch.cuda.synchronize()
        for b, yw, yn in zip(bws, y_ws, y_na):
            assert torch.equal(yw, yn)
            p, s, g = oracle.quantize(b)
            yr, l1 = oracle.gemv(bx, p, s, g, threads=8)
            ok, worst = oracle.tolerance_ok(yn.cpu().numpy().astype(np.float64), yr, l1)
            assert ok, worst
    # more scratch than the array holds: 17 chunks x 1088 pairs of partial sums (18.9 MB)
    A = 1 << 20
    big = (fp4._Proj * 1)(fp4._Proj(A, None, A, 17408, A, 17408))
    assert fp4.workspace_bytes(fp4.OP_GEMV, 8, 17408, [17408]) > 16 << 20
    assert L.fp4_gemv_multi_noalloc(big, 1, A, 8, 17408, stream) == -7
