"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Quantiser bytes and re-tiled layouts must be bit-exact. Products must satisfy
|y_gpu - y_ref| <= 2e-3 * sum_k |w_nk * x_k| per output element (y_ref in
fp64, w the dequantised weight), and exactly equal where every partial sum is
exact in fp32. Sizes run from single tiles with ragged tails to the full
workload shapes, all through the C ABI (via the thin binding)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_to_float32, float32_to_bf16_bits, bf16_tensor, fp8_release, norm_gain

from gpu_common import (THREADS, act_bits, assert_within_tolerance, dev, gpu_u8, oracle_quant, to_gpu_bf16,
                        weight_bits)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import bit_block_scaled_fp4_amd as fp4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_quant(bits, layout="tiled"):
    w = fp4.quantize(to_gpu_bf16(bits), layout)
    torch.cuda.synchronize()
    return w


def check_quant_bytes(bits, what):
    p, s, g = oracle.quantize(bits)
    w = gpu_quant(bits, "rowmajor")
    gp, gsc, gg = gpu_u8(w.packed), gpu_u8(w.scales), w.gscale.item()
    assert np.float32(gg) == g, (what, gg, g)
    assert np.array_equal(gsc.reshape(s.shape), s), (what, np.flatnonzero(gsc.reshape(s.shape) != s)[:8])
    assert np.array_equal(gp.reshape(p.shape), p), (what, np.flatnonzero(gp.reshape(p.shape) != p)[:8])
    wt = gpu_quant(bits, "tiled")
    assert np.array_equal(gpu_u8(wt.packed), oracle.tile(p, s)), what
    assert wt.gscale.item() == gg
    return p, s, g


# ------------------------------------------------------------------- quantiser
def edge_tensors():
    rng = np.random.default_rng(11)
    out = {}
    from test_oracle_pins import load_worked_example
    out["worked_example"] = load_worked_example()[0]
    out["zeros"] = np.zeros((9, 48), np.uint16)
    out["ragged_11x48"] = bf16_tensor((11, 48), 7, 0.1)
    out["ragged_13x1040"] = bf16_tensor((13, 1040), 8, 0.02, outlier_p=0.01, outlier_scale=20)
    out["one_row_16"] = bf16_tensor((1, 16), 9, 3.0)
    out["tiny"] = float32_to_bf16_bits(rng.normal(0, 1e-30, (16, 64)).astype(np.float32))
    out["huge"] = float32_to_bf16_bits(rng.normal(0, 1e30, (16, 64)).astype(np.float32))
    wide = rng.normal(0, 1, (32, 256)) * np.exp(rng.uniform(-20, 5, (32, 256)))
    out["wide_dynamic_range"] = float32_to_bf16_bits(wide.astype(np.float32))
    ties = np.array([oracle.e2m1_value(c) for c in range(16)])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5])
    v = rng.choice(np.concatenate([ties, mids, -mids]), (24, 128)) * 0.4375   # exact tie points for d = 0.4375
    v[:, ::16] = 2.625
    out["ties"] = float32_to_bf16_bits(v.astype(np.float32))
    neg = -np.abs(rng.normal(0, 1, (8, 64))) * 1e-3
    neg[:, 0] = 5.0
    out["small_negatives"] = float32_to_bf16_bits(neg.astype(np.float32))
    return out


@pytest.mark.parametrize("name", list(edge_tensors().keys()))
def test_quantize_bit_exact_edge_cases(name):
    print("quantize edge case", name, flush=True)
    check_quant_bytes(edge_tensors()[name], name)


@pytest.mark.parametrize("name", list(edge_tensors().keys()))
def test_products_on_edge_tensors(name):
    """The decode products and the prefill on the quantiser's edge tensors
    (rounding ties, zeros, tiny ~1e-30 and huge ~1e30 weights, a wide dynamic
    range, ragged shapes, the worked example): 1 row on the vector ALUs, 3 and
    8 rows on the 8-row matrix-core kernel with and without a workspace, 12
    rows on the 16-row kernel, 37 rows through the prefill. Every result
    within the tolerance of the oracle (products of zero rows exactly 0)."""
    bw = edge_tensors()[name]
    N, K = bw.shape
    print("edge products", name, N, K, flush=True)
    w = gpu_quant(bw)
    p, s, g = oracle.quantize(bw)
    for M in (1, 3, 8, 12, 37):
        bx = bf16_tensor((M, K), 6500 + M + N, 1.0)
        x = to_gpu_bf16(bx)
        yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
        if M == 37:
            got = [("prefill", fp4.gemm_prefill(x, w))]
        else:
            work = ws_for(fp4.OP_GEMV, M, K, [N])
            got = [("gemv", fp4.gemv(x, w)), ("gemv ws", fp4.gemv(x, w, workspace=work))]
        torch.cuda.synchronize()
        for what, y in got:
            assert_within_tolerance(y.cpu().numpy(), yr, l1, "edge %s %s M=%d" % (name, what, M))


@pytest.mark.parametrize("wl,t", [("gemv_1024", "w"), ("qwen3_0p6b_decode", "L1.q"), ("qwen3_0p6b_decode", "L1.o"),
                                  ("qwen3_0p6b_decode", "L28.down"), ("dense27b_layer", "gate"),
                                  ("dense27b_layer", "up"), ("dense27b_layer", "down"), ("lm_head", "w")])
def test_quantize_bit_exact_workloads(wl, t):
    print("quantize", wl, t, flush=True)
    p, s, g = check_quant_bytes(weight_bits(wl, t), "%s/%s" % (wl, t))
    op, os_, og = oracle_quant(wl, t)
    assert og == g


# ------------------------------------------------------ quantiser, FP8 source
def check_quant_fp8(codes, scale, what):
    p, s, g = oracle.quantize_fp8(codes, scale)
    C = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(dev())
    S = torch.tensor([float(scale)], dtype=torch.float32, device=dev())
    w = fp4.quantize_fp8(C, S, "rowmajor")
    torch.cuda.synchronize()
    gp, gsc, gg = gpu_u8(w.packed), gpu_u8(w.scales), w.gscale.item()
    assert np.float32(gg) == g, (what, gg, g)
    assert np.array_equal(gsc.reshape(s.shape), s), (what, np.flatnonzero(gsc.reshape(s.shape) != s)[:8])
    assert np.array_equal(gp.reshape(p.shape), p), (what, np.flatnonzero(gp.reshape(p.shape) != p)[:8])
    wt = fp4.quantize_fp8(C.view(torch.float8_e4m3fn), S, "tiled")
    torch.cuda.synchronize()
    assert np.array_equal(gpu_u8(wt.packed), oracle.tile(p, s)), what
    assert wt.gscale.item() == gg


def fp8_edge_cases():
    rng = np.random.default_rng(23)
    every = np.arange(256, dtype=np.uint8)
    every = every[(every & 0x7F) != 0x7F]                       # all 254 non-NaN codes
    out = {
        "ragged_13x1040": fp8_release((13, 1040), 21, 0.02, outlier_p=0.01, outlier_scale=20),
        "one_row_16": fp8_release((1, 16), 22, 1.0),
        "every_code_pow2_scale": (np.resize(rng.permutation(every), (16, 1024)), np.float32(2.0 ** -7)),
        "every_code_odd_scale": (np.resize(rng.permutation(every), (16, 1024)), np.float32(0.0137)),
        "negative_scale": (np.resize(every, (8, 512)), np.float32(-0.5)),
        "zero_scale": (np.resize(every, (8, 512)), np.float32(0.0)),
        "subnormal_codes_only": ((rng.integers(0, 8, (24, 128)) | (rng.integers(0, 2, (24, 128)) << 7)).astype(np.uint8),
                                 np.float32(0.3)),
        "tiny_scale": (np.resize(every, (8, 256)), np.float32(1e-30)),
        "huge_scale": (np.resize(every, (8, 256)), np.float32(3e35)),
    }
    return out


@pytest.mark.parametrize("name", list(fp8_edge_cases().keys()))
def test_quantize_fp8_bit_exact_edge_cases(name):
    print("quantize fp8 edge case", name, flush=True)
    codes, scale = fp8_edge_cases()[name]
    check_quant_fp8(codes, scale, name)


@pytest.mark.parametrize("shape,seed", [((1024, 1024), 31), ((5120, 17408), 32)])
def test_quantize_fp8_bit_exact_workload(shape, seed):
    """An FP8 release of the 1024 x 1024 and 27B down-projection shapes
    (N(0, 0.015) weights with 0.1 % outliers x20, like the bf16 workloads)."""
    print("quantize fp8 workload", shape, flush=True)
    codes, scale = fp8_release(shape, seed, 0.015, outlier_p=0.001, outlier_scale=20)
    check_quant_fp8(codes, scale, "fp8 %dx%d" % shape)


def test_retile_bit_exact_and_pads_with_zeros():
    for shape, seed in [((11, 1040), 3), ((24, 3072), 4), ((5, 16), 5), ((300, 2064), 6)]:
        bits = bf16_tensor(shape, seed, 0.05)
        w = gpu_quant(bits, "rowmajor")
        N, K = shape
        pb, _ = fp4.layout_bytes(N, K, "tiled")
        out = fp4.NVFP4Weight(torch.full((pb,), 0xAB, dtype=torch.uint8, device=dev()), None, w.gscale, N, K,
                              fp4.TILED)
        fp4.retile(w, out)
        p, s, _ = oracle.quantize(bits)
        assert np.array_equal(gpu_u8(out.packed), oracle.tile(p, s)), shape


# ------------------------------------------------------------------- products
def run_gemv(bits_w, bits_x):
    w = gpu_quant(bits_w)
    y = fp4.gemv(to_gpu_bf16(bits_x), w)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("N,K,M", [(1, 16, 1), (7, 32, 1), (16, 1024, 1), (1000, 1040, 1), (1000, 1040, 2),
                                   (333, 2064, 3), (17, 3072, 5), (64, 5120, 8), (130, 17408, 4), (40, 8192, 16),
                                   (257, 1024, 7), (2050, 2048, 1), (300, 1040, 5), (97, 2064, 17),
                                   (520, 3072, 32), (130, 4096, 40), (64, 1024, 64),
                                   # M = 1 with more than 16 chunks: about one workgroup per CU, every
                                   # wave streaming several chunks (1 and 2 row groups per workgroup)
                                   (100, 17424, 1), (3000, 20480, 1),
                                   # several row groups per workgroup, each over several rounds: the
                                   # workgroup's tiles go round-robin over its waves (a ragged last
                                   # workgroup with one valid group; M = 2 and 4 with three and five chunks)
                                   (2056, 17472, 1), (4100, 3008, 2), (4104, 5120, 4),
                                   # M = 2..4 with at least 8 chunks: one row group of 8 waves per
                                   # workgroup, waves taking chunks j, j + 8, ... (a ragged K tail;
                                   # 17 chunks and a partial last row group)
                                   (300, 8208, 2), (9, 16400, 3),
                                   # 9 to 16 rows over 17, 25 and 40 chunks without a workspace (atomic adds)
                                   (56, 17408, 10), (24, 25600, 16), (40, 40960, 12)])
def test_gemv_small_shapes(N, K, M):
    print("gemv", N, K, M, flush=True)
    bw = bf16_tensor((N, K), N * 7 + K, 0.03, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 99 + M, 1.0)
    y = run_gemv(bw, bx)
    p, s, g = oracle.quantize(bw)
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y, yr, l1, "gemv %dx%d M=%d" % (N, K, M))


@pytest.mark.parametrize("N,K,Ms", [(16, 1 << 20, (1, 5)), ((1 << 21) - 8, 16, (1, 3))])
def test_extreme_shapes(N, K, Ms):
    """Near the size limits: K = 2^20 (1024 chunks per row group: 4.7 MB of
    tiles per group, one workgroup streaming them) and N = 2^21 - 8 rows
    (262143 row groups; the prefill's 256-row output slab just under 2 GB).
    Quantisation bit-exact; the decode product and the prefill product
    within the tolerance."""
    print("extreme", N, K, Ms, flush=True)
    bw = bf16_tensor((N, K), 4 * N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    p, s, g = check_quant_bytes(bw, "extreme %dx%d" % (N, K))
    w = gpu_quant(bw)
    for M in Ms:
        bx = bf16_tensor((M, K), 17 + M, 1.0)
        x = to_gpu_bf16(bx)
        yg = fp4.gemv(x, w)
        yp = fp4.gemm_prefill(x, w)
        torch.cuda.synchronize()
        yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
        assert_within_tolerance(yg.cpu().numpy(), yr, l1, "extreme gemv %dx%d M=%d" % (N, K, M))
        assert_within_tolerance(yp.cpu().numpy(), yr, l1, "extreme prefill %dx%d M=%d" % (N, K, M))


@pytest.mark.parametrize("M", [3, 6, 12])
def test_gemv_exact_when_every_partial_sum_is_exact(M):
    """Every block holds 2.625 (so all scales are 0x7E and gscale = 2^-10) and
    x is +-2^k: every product and partial sum, in any order, is exact in fp32
    (multiples of 2^-4 below 2^17, times 448), so the GPU result must equal
    the exact oracle value bit for bit. M = 3: vector ALUs; 6: the block-split
    matrix-core kernel; 12: the 16-row one (both with the K-chunk reduce)."""
    rng = np.random.default_rng(21)
    N, K = 48, 2048
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6]) * 0.4375
    W = rng.choice(mags, (N, K)) * rng.choice([-1, 1], (N, K))
    W[:, ::16] = 2.625
    bw = float32_to_bf16_bits(W.astype(np.float32))
    x = (2.0 ** rng.integers(-3, 4, (M, K))) * rng.choice([-1, 1], (M, K))
    bx = float32_to_bf16_bits(x.astype(np.float32))
    y = run_gemv(bw, bx)
    p, s, g = oracle.quantize(bw)
    assert g == 2.0 ** -10 and np.all(s == 0x7E)
    yr, _ = oracle.gemv(bx, p, s, g)
    assert np.array_equal(y.astype(np.float64), yr)
    w = gpu_quant(bw)
    yp = fp4.gemm_prefill(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    assert np.array_equal(yp.cpu().numpy().astype(np.float64), yr)


@pytest.mark.parametrize("M", [3, 5, 8, 12])
def test_gemv_block_scales_alternate_by_parity(M):
    """Even 16-element blocks are 1000 times smaller than odd ones, with the
    ratio varied per row, so a block scale applied to the other block of its
    piece (the matrix-core kernels handle the two blocks of a 32-element
    piece in different rows or lanes) moves y far outside the tolerance."""
    rng = np.random.default_rng(23 + M)
    N, K = 40, 3072
    W = rng.normal(0, 1, (N, K))
    parity = (np.arange(K) // 16) % 2
    W *= np.where(parity == 0, 1e-3, 1.0)[None, :] * rng.uniform(0.5, 2.0, (N, 1))
    bw = float32_to_bf16_bits(W.astype(np.float32))
    bx = float32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
    y = run_gemv(bw, bx)
    p, s, g = oracle.quantize(bw)
    yr, l1 = oracle.gemv(bx, p, s, g)
    assert_within_tolerance(y, yr, l1, "alternating block scales M=%d" % M)


def test_gemv_one_hot_selects_a_column():
    """x = e_k returns column k of the dequantised weight: pins the nibble
    order, the block-scale index and the tiled layout on the GPU."""
    bw = weight_bits("gemv_1024", "w")[:200]
    p, s, g = oracle.quantize(bw)
    D = oracle.dequant(p, s, g)
    w = gpu_quant(bw)
    ks = [0, 1, 2, 15, 16, 31, 32, 33, 511, 512, 1000, 1023]
    X = np.zeros((len(ks), 1024), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    y = fp4.gemv(to_gpu_bf16(float32_to_bf16_bits(X)), w)
    torch.cuda.synchronize()
    # E2M1*E4M3 is exact in fp32, so the only rounding is the final product
    # with gscale: the result is the exact dequantised weight rounded to fp32.
    assert np.array_equal(y.cpu().numpy(), D[:, ks].T.astype(np.float32))


def test_gemv_workload_gemv_1024():
    bw, bx = weight_bits("gemv_1024", "w"), act_bits("gemv_1024", "x")
    y = run_gemv(bw, bx)
    p, s, g = oracle_quant("gemv_1024", "w")
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y, yr, l1, "gemv_1024")


def test_gemv_workload_qwen_decode_all_layers():
    """28 layers x (fused QKV, O, fused gate_up, down) at M=1."""
    wl = "qwen3_0p6b_decode"
    for l in range(1, 29):
        print("layer", l, flush=True)
        xs = {k: act_bits(wl, "L%d.x%d" % (l, k)) for k in (1024, 2048, 3072)}
        ws = {t: gpu_quant(weight_bits(wl, "L%d.%s" % (l, t))) for t in ("q", "k", "v", "o", "gate", "up", "down")}
        x1 = to_gpu_bf16(xs[1024])
        qkv = torch.empty((1, 4096), dtype=torch.float32, device=dev())
        fp4.gemv_multi(x1, [ws["q"], ws["k"], ws["v"]], [qkv, qkv[:, 2048:], qkv[:, 3072:]], [4096] * 3)
        gu = torch.empty((1, 6144), dtype=torch.float32, device=dev())
        fp4.gemv_multi(x1, [ws["gate"], ws["up"]], [gu, gu[:, 3072:]], [6144] * 2)
        o = fp4.gemv(to_gpu_bf16(xs[2048]), ws["o"])
        d = fp4.gemv(to_gpu_bf16(xs[3072]), ws["down"])
        torch.cuda.synchronize()
        res = {"q": qkv[:, :2048], "k": qkv[:, 2048:3072], "v": qkv[:, 3072:], "gate": gu[:, :3072],
               "up": gu[:, 3072:], "o": o, "down": d}
        xin = {"q": 1024, "k": 1024, "v": 1024, "gate": 1024, "up": 1024, "o": 2048, "down": 3072}
        for t, yt in res.items():
            p, s, g = oracle_quant(wl, "L%d.%s" % (l, t))
            assert gpu_u8(ws[t].gscale)[0] == g
            yr, l1 = oracle.gemv(xs[xin[t]], p, s, g, threads=THREADS)
            assert_within_tolerance(yt.cpu().numpy(), yr, l1, "L%d.%s" % (l, t))


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_gemv_workload_dense27b(M):
    """gate_up (one fused launch) and down of the 27B-class layer; M=1 is the
    single-stream decode layer, M in {2,4,8,16} the small-M batch."""
    wl = "dense27b_layer"
    print("dense27b M=%d" % M, flush=True)
    if M == 1:
        xin, xmid = act_bits(wl, "x_in"), act_bits(wl, "x_mid")
    else:
        xin, xmid = act_bits("dense27b_smallm", "x_in_m%d" % M), act_bits("dense27b_smallm", "x_mid_m%d" % M)
    wg, wu, wd = (gpu_quant(weight_bits(wl, t)) for t in ("gate", "up", "down"))
    gu = torch.empty((M, 2 * 17408), dtype=torch.float32, device=dev())
    fp4.gemv_multi(to_gpu_bf16(xin), [wg, wu], [gu, gu[:, 17408:]], [2 * 17408] * 2)
    yd = fp4.gemv(to_gpu_bf16(xmid), wd)
    torch.cuda.synchronize()
    gu = gu.cpu().numpy()
    for t, yt, xx in (("gate", gu[:, :17408], xin), ("up", gu[:, 17408:], xin), ("down", yd.cpu().numpy(), xmid)):
        p, s, g = oracle_quant(wl, t)
        yr, l1 = oracle.gemv(xx, p, s, g, threads=THREADS)
        assert_within_tolerance(yt, yr, l1, "%s M=%d" % (t, M))


@pytest.mark.parametrize("M", [1, 8])
def test_gemv_workload_lm_head(M):
    bw, bx = weight_bits("lm_head", "w"), act_bits("lm_head", "x_m%d" % M)
    w = gpu_quant(bw)
    y = fp4.gemv(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s, g = oracle_quant("lm_head", "w")
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "lm_head M=%d" % M)


@pytest.mark.parametrize("M", [3, 4])
def test_gemv_lm_head_three_and_four_rows(M):
    """3 or 4 rows on a call of at least 32 MiB go to
    the matrix cores (the LM head: one chunk, 87 MB); the rows are the first
    M of the LM head's 8-row activations."""
    bw, bx = weight_bits("lm_head", "w"), act_bits("lm_head", "x_m8")[:M]
    w = gpu_quant(bw)
    y = fp4.gemv(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s, g = oracle_quant("lm_head", "w")
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "lm_head M=%d" % M)


@pytest.mark.parametrize("M", [12, 16])
def test_gemv_lm_head_twelve_and_sixteen_rows(M):
    """9 to 16 rows of the LM head run the 16-row matrix-core kernel on its
    one K chunk, writing y without chunk sums. Its launch plan gives each
    wave five pairs, an odd count, so the pair loop (two register sets in
    turn) ends halfway through its last iteration. Activations: seeded N(0, 1)
    rows of the LM head's width."""
    bw, bx = weight_bits("lm_head", "w"), bf16_tensor((M, 1024), 430 + M, 1.0)
    w = gpu_quant(bw)
    y = fp4.gemv(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s, g = oracle_quant("lm_head", "w")
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "lm_head M=%d" % M)


def test_gemv_multi_equals_oracle_for_each_projection_and_is_deterministic():
    rng_shapes = [(2048, 1024), (1024, 1024), (1024, 1024), (333, 1024)]
    ws, bws = [], []
    for i, (N, K) in enumerate(rng_shapes):
        b = bf16_tensor((N, K), 500 + i, 0.02)
        bws.append(b)
        ws.append(gpu_quant(b))
    bx = bf16_tensor((3, 1024), 77, 1.0)
    x = to_gpu_bf16(bx)
    outs = [torch.empty((3, N), dtype=torch.float32, device=dev()) for N, _ in rng_shapes]
    fp4.gemv_multi(x, ws, outs)
    outs2 = [torch.empty_like(o) for o in outs]
    fp4.gemv_multi(x, ws, outs2)
    torch.cuda.synchronize()
    for b, o, o2 in zip(bws, outs, outs2):
        p, s, g = oracle.quantize(b)
        yr, l1 = oracle.gemv(bx, p, s, g)
        assert_within_tolerance(o.cpu().numpy(), yr, l1, "multi")
        assert torch.equal(o, o2)


def ws_for(op, M, K, Ns):
    return fp4.new_workspace(fp4.workspace_bytes(op, M, K, Ns), dev())


@pytest.mark.parametrize("M", [5, 8, 9])
def test_gemv_multi_matrix_core_ragged_projections(M):
    """Several projections of unequal, ragged row counts (333, 16, 1000 rows;
    K = 3008: three chunks, so the K split runs) in one launch on the
    matrix-core path (M >= 5; M = 9 stages 16 activation rows, M = 5 and 8
    eight), each equal to the oracle within the tolerance: with a workspace
    (chunk partials added in chunk order, for 8-row passes inside the launch
    by the last workgroup of each pair block to arrive, for 16-row passes by a
    second kernel: repeatable bit for bit, the counter header left at zero)
    and without (y zeroed, then atomic adds; outputs start as NaN)."""
    print("gemv_multi mfma", M, flush=True)
    Ns, K = (333, 16, 1000), 3008
    bws = [bf16_tensor((N, K), 800 + N, 0.02, outlier_p=0.002, outlier_scale=20.0) for N in Ns]
    ws = [gpu_quant(b) for b in bws]
    bx = bf16_tensor((M, K), 900 + M, 1.0)
    x = to_gpu_bf16(bx)
    work = ws_for(fp4.OP_GEMV, M, K, Ns)
    assert work.numel() > 65536
    outs = [torch.empty((M, N), dtype=torch.float32, device=dev()) for N in Ns]
    outs2 = [torch.empty_like(o) for o in outs]
    outs_na = [torch.full_like(o, float("nan")) for o in outs]
    fp4.gemv_multi(x, ws, outs, workspace=work)
    fp4.gemv_multi(x, ws, outs2, workspace=work)
    fp4.gemv_multi(x, ws, outs_na)
    torch.cuda.synchronize()
    assert torch.count_nonzero(work[:65536]) == 0        # the counter header stays zero
    for b, o, o2, on in zip(bws, outs, outs2, outs_na):
        p, s, g = oracle.quantize(b)
        yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
        assert_within_tolerance(o.cpu().numpy(), yr, l1, "multi mfma ws M=%d" % M)
        assert_within_tolerance(on.cpu().numpy(), yr, l1, "multi mfma atomic M=%d" % M)
        assert torch.equal(o, o2)


@pytest.mark.parametrize("N,K,M", [(56, 17408, 10), (24, 25600, 16), (40, 40960, 12), (30, 5120, 9)])
def test_gemv_chunk_sums_16_rows(N, K, M):
    """16-row matrix-core passes with a workspace: the second kernel adds all
    chunk partials of an output in chunk order, loading 8, 16, 24 or 32 of
    them per round (5, 17, 25 chunks: one round; 40: two rounds of 32, the
    second clamped). Within the tolerance of the oracle, repeatable bit for
    bit, the counter header left at zero."""
    print("chunk sums", N, K, M, flush=True)
    bw = bf16_tensor((N, K), 3 * N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 70 + M, 1.0)
    w = gpu_quant(bw)
    x = to_gpu_bf16(bx)
    work = ws_for(fp4.OP_GEMV, M, K, [N])
    y = fp4.gemv(x, w, workspace=work)
    y2 = fp4.gemv(x, w, workspace=work)
    torch.cuda.synchronize()
    assert torch.count_nonzero(work[:65536]) == 0
    assert torch.equal(y, y2)
    p, s, g = oracle.quantize(bw)
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "chunk sums %dx%d M=%d" % (N, K, M))


@pytest.mark.parametrize("N,K,M", [(131072, 1040, 6), (4100, 17408, 4)])
def test_gemv_chunk_sums_8_rows(N, K, M):
    """Passes of at most 8 rows with a workspace. 131072 x 1040 at 6 rows has
    more pair blocks (1024 of 8 pairs) than the workspace header has arrival
    counters (512), so its chunk sums (2 chunks, the second 16 wide) go to
    the second kernel; 4100 x 17408 at 4 rows adds its 17 chunks inside the
    launch (the
    last workgroup of each pair block, three rounds of loads through one
    buffer resource, a partial last pair). Within the tolerance of the
    oracle, repeatable bit for bit, the counter header left at zero."""
    print("chunk sums", N, K, M, flush=True)
    bw = bf16_tensor((N, K), 5 * N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 80 + M, 1.0)
    w = gpu_quant(bw)
    x = to_gpu_bf16(bx)
    work = ws_for(fp4.OP_GEMV, M, K, [N])
    y = fp4.gemv(x, w, workspace=work)
    y2 = fp4.gemv(x, w, workspace=work)
    torch.cuda.synchronize()
    assert torch.count_nonzero(work[:65536]) == 0
    assert torch.equal(y, y2)
    p, s, g = oracle.quantize(bw)
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "chunk sums %dx%d M=%d" % (N, K, M))


def test_workspace_too_small_is_an_error():
    """A workspace smaller than fp4_workspace_bytes reports is rejected before
    any launch; one that is large enough but not 256-byte aligned too."""
    N, K, M = 1000, 3008, 8
    w = gpu_quant(bf16_tensor((N, K), 5, 0.02))
    x = to_gpu_bf16(bf16_tensor((M, K), 6, 1.0))
    need = fp4.workspace_bytes(fp4.OP_GEMV, M, K, [N])
    small = fp4.new_workspace(need - 1, dev())
    with pytest.raises(fp4.Fp4Error) as e:
        fp4.gemv(x, w, workspace=small)
    assert e.value.status == -7
    big = fp4.new_workspace(need + 512, dev())
    L = fp4.raw()
    y = torch.empty((M, N), dtype=torch.float32, device=dev())
    st = L.fp4_gemv_ws(y.data_ptr(), x.data_ptr(), w.packed.data_ptr(), None, w.gscale.data_ptr(), M, N, K,
                       big.data_ptr() + 16, need, torch.cuda.current_stream().cuda_stream)
    assert st == -3


# --------------------------------------------------------------------- prefill
# (300, 16452, 80) and (257, 16400, 1040) take 256 x 192 tiles, (300, 32768, 80) takes 256 x 256 tiles
@pytest.mark.parametrize("M,N,K", [(1, 8, 16), (37, 300, 1040), (200, 129, 2048), (128, 256, 64), (300, 1000, 5120),
                                   (513, 136, 1984), (64, 64, 80), (300, 16452, 80), (257, 16400, 1040),
                                   (300, 32768, 80)])
def test_prefill_small_shapes(M, N, K):
    print("prefill", M, N, K, flush=True)
    bw = bf16_tensor((N, K), M + N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 3 * M + 1, 1.0)
    w = gpu_quant(bw)
    y = fp4.gemm_prefill(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s, g = oracle.quantize(bw)
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "prefill %d %d %d" % (M, N, K))


@pytest.mark.parametrize("M,K,Ns", [(300, 1040, (300, 8, 1000)), (37, 80, (16452, 16400)), (513, 2048, (129,)),
                                    (257, 64, (256, 128, 192, 8, 200, 1000, 64, 72))])
def test_prefill_multi_column_slices(M, K, Ns):
    """Several projections in one launch, each writing a column slice of one
    shared [M][ldy] output (ldy = sum of N + 3 guard columns): every slice
    is within the tolerance of the oracle, as is the separate
    fp4_gemm_prefill result, a second launch repeats the first bit for bit,
    and the guard columns are never written. (Fused and separate launches
    may split different tiles along K, so they agree to rounding only.)"""
    print("prefill_multi", M, K, Ns, flush=True)
    bx = bf16_tensor((M, K), 11 * M + K, 1.0)
    x = to_gpu_bf16(bx)
    bws = [bf16_tensor((N, K), 900 + 7 * i + N, 0.02, outlier_p=0.002, outlier_scale=20.0) for i, N in enumerate(Ns)]
    ws = [gpu_quant(b) for b in bws]
    ldy = sum(Ns) + 3
    y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device=dev())
    offs = np.cumsum((0,) + tuple(Ns))
    fp4.gemm_prefill_multi(x, ws, [y[:, o:] for o in offs[:-1]], [ldy] * len(Ns))
    y2 = torch.full_like(y, float("nan"))
    fp4.gemm_prefill_multi(x, ws, [y2[:, o:] for o in offs[:-1]], [ldy] * len(Ns))
    sep = [fp4.gemm_prefill(x, w) for w in ws]
    torch.cuda.synchronize()
    assert torch.isnan(y[:, offs[-1]:]).all()
    assert torch.equal(y[:, :offs[-1]], y2[:, :offs[-1]])
    for i, (b, N) in enumerate(zip(bws, Ns)):
        part = y[:, offs[i]:offs[i] + N]
        p, s, g = oracle.quantize(b)
        yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
        assert_within_tolerance(part.cpu().numpy(), yr, l1, "prefill_multi %d" % i)
        assert_within_tolerance(sep[i].cpu().numpy(), yr, l1, "prefill separate %d" % i)


# Shapes whose last round of tiles is split along K after a full round of
# whole tiles (two launches): 300 x 32776 x 1040 takes 342 tiles of 256 x 192
# (the last 86, in token rows 256..299, in 2 K ranges); 513 x 32648 x 1040
# takes 384 tiles of 256 x 256 (the last 128, token row 512, in 2 K ranges).
@pytest.mark.parametrize("M,N,K,rows", [(300, 32776, 1040, [0, 1, 100, 255, 256, 257, 280, 299]),
                                        (513, 32648, 1040, [0, 255, 256, 300, 511, 512])])
def test_prefill_whole_and_split_tiles(M, N, K, rows):
    print("prefill whole+split", M, N, K, flush=True)
    bw = bf16_tensor((N, K), 7 * N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 5 * M + 3, 1.0)
    w = gpu_quant(bw)
    x = to_gpu_bf16(bx)
    work = ws_for(fp4.OP_GEMM_PREFILL, M, K, [N])
    assert work.numel() > 65536                          # the last round is split
    y = fp4.gemm_prefill(x, w, workspace=work)
    y2 = fp4.gemm_prefill(x, w, workspace=work)
    y3 = fp4.gemm_prefill(x, w)                          # no workspace: nothing split
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.count_nonzero(work[:65536]) == 0
    p, s, g = oracle.quantize(bw)
    yr, l1 = oracle.gemv(bx[rows], p, s, g, threads=THREADS)
    assert_within_tolerance(y[rows].cpu().numpy(), yr, l1, "prefill whole+split %d %d %d" % (M, N, K))
    assert_within_tolerance(y3[rows].cpu().numpy(), yr, l1, "prefill unsplit %d %d %d" % (M, N, K))


def test_prefill_full_size_sampled_rows():
    """M=2048 tokens x gate_up 34816x5120 (two 17408-row tensors in one
    [2048][34816] output via two calls into column slices is not possible with
    ldy = N, so each half is its own call). Checked on 8 sampled token rows,
    all 34816 outputs each."""
    wl = "prefill"
    bx = act_bits(wl, "x")
    x = to_gpu_bf16(bx)
    rows = [0, 1, 127, 128, 1000, 1500, 2046, 2047]
    ws, ys = {}, {}
    for t in ("gate", "up"):
        w = ws[t] = gpu_quant(weight_bits("dense27b_layer", t))
        y = ys[t] = fp4.gemm_prefill(x, w)
        y2 = fp4.gemm_prefill(x, w)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        p, s, g = oracle_quant("dense27b_layer", t)
        yr, l1 = oracle.gemv(bx[rows], p, s, g, threads=THREADS)
        assert_within_tolerance(y[rows].cpu().numpy(), yr, l1, "prefill %s" % t)
    # the fused launch the bench times: gate and up into the halves of one
    # [2048][34816] output; its last round of tiles is split along K
    N = ws["gate"].N
    yf = torch.empty((2048, 2 * N), dtype=torch.float32, device=dev())
    yf2 = torch.empty_like(yf)
    work = ws_for(fp4.OP_GEMM_PREFILL, 2048, 5120, [N, N])
    for out in (yf, yf2):
        fp4.gemm_prefill_multi(x, [ws["gate"], ws["up"]], [out[:, :N], out[:, N:]], [2 * N, 2 * N], workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(yf, yf2)
    # the split tiles are the last ones: token slab 7 (rows 1792..2047), the last 64 x 256 columns of up
    rows_f = rows + [1792, 1900]
    for h, t in enumerate(("gate", "up")):
        p, s, g = oracle_quant("dense27b_layer", t)
        yr, l1 = oracle.gemv(bx[rows_f], p, s, g, threads=THREADS)
        assert_within_tolerance(yf[rows_f, h * N:(h + 1) * N].cpu().numpy(), yr, l1, "prefill fused %s" % t)


def test_gemv_and_prefill_agree_with_each_other():
    bw = weight_bits("gemv_1024", "w")
    w = gpu_quant(bw)
    bx = bf16_tensor((16, 1024), 4242, 1.0)
    x = to_gpu_bf16(bx)
    a, b = fp4.gemv(x, w), fp4.gemm_prefill(x, w)
    torch.cuda.synchronize()
    p, s, g = oracle_quant("gemv_1024", "w")
    yr, l1 = oracle.gemv(bx, p, s, g)
    assert_within_tolerance(a.cpu().numpy(), yr, l1, "gemv")
    assert_within_tolerance(b.cpu().numpy(), yr, l1, "prefill")


def test_errors_raise_on_gpu():
    W = torch.zeros((8, 24), dtype=torch.bfloat16, device=dev())
    with pytest.raises(fp4.Fp4Error):
        fp4.quantize(W, out=fp4.NVFP4Weight(torch.zeros(64, dtype=torch.uint8, device=dev()),
                                            torch.zeros(64, dtype=torch.uint8, device=dev()),
                                            torch.zeros(1, device=dev()), 8, 24))


# ------------------------------------------------------------- greedy choice
def planted_rows(M, N, seed):
    """fp32 rows with the cases the order rule decides: ties of the maximum,
    NaNs, signed zeros, infinities, a constant row, an all -inf row."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((M, N)).astype(np.float32)
    for m in range(M):
        kind = m % 7
        if kind == 1:                                   # the maximum at up to three places
            y[m, rng.choice(N, size=min(3, N), replace=False)] = y[m].max() + 1.0
        elif kind == 2:                                 # two NaNs: the first wins
            a, b = sorted(rng.choice(N, size=2, replace=N < 2))
            y[m, a] = np.nan
            y[m, b] = np.float32(-np.nan)
        elif kind == 3:                                 # only signed zeros: index 0
            y[m] = np.where(rng.random(N) < 0.5, np.float32(-0.0), np.float32(0.0))
        elif kind == 4:                                 # +inf twice
            y[m, rng.choice(N, size=min(2, N), replace=False)] = np.inf
        elif kind == 5:                                 # a constant row
            y[m] = np.float32(0.25)
        elif kind == 6:
            y[m] = -np.inf
    return y


# segments of 4096 elements per workgroup: one, exactly one, one plus one,
# several with a ragged tail, the vocabulary size, a long row
@pytest.mark.parametrize("M,N", [(1, 1), (7, 31), (7, 4096), (7, 4097), (9, 3 * 4096 + 5), (8, 151936),
                                 (2, 1 << 20)])
def test_argmax_rows_bit_exact(M, N):
    y = planted_rows(M, N, seed=M * 1000003 + N)
    yt = torch.from_numpy(y).to(dev())
    work = ws_for(fp4.OP_ARGMAX_ROWS, M, 0, [N])
    got = fp4.argmax_rows(yt, workspace=work).cpu().numpy()
    got_nows = fp4.argmax_rows(yt).cpu().numpy()
    ref = oracle.argmax_rows(y)
    assert np.array_equal(got, ref)
    assert np.array_equal(got_nows, ref)


def test_argmax_rows_strided_and_repeated():
    """Row stride above N through the C ABI; repeated launches of different
    sizes sharing one workspace (the per-row counters must come back to zero
    every time), more rows than the workspace header has counters (600: two
    launches), and the same calls without a workspace."""
    L = fp4.raw()
    stream = torch.cuda.current_stream().cuda_stream
    cases = [(3, 10000, 10007), (8, 151936, 151936), (3, 10000, 10007), (40, 9000, 9001), (1, 4097, 4100),
             (600, 5000, 5003), (3, 10000, 10007)]
    work = fp4.new_workspace(max(fp4.workspace_bytes(fp4.OP_ARGMAX_ROWS, M, 0, [N]) for M, N, _ in cases), dev())
    for M, N, ldy in cases:
        y = planted_rows(M, ldy, seed=N + ldy + M)
        y[:, N:] = np.inf                                # past N: must be ignored
        ref = oracle.argmax_rows(np.ascontiguousarray(y[:, :N]))
        yt = torch.from_numpy(y).to(dev())
        for wp, wb in ((work.data_ptr(), work.numel()), (None, 0)):
            idx = torch.full((M,), -1, dtype=torch.int32, device=dev())
            assert L.fp4_argmax_rows(idx.data_ptr(), yt.data_ptr(), M, N, ldy, wp, wb, stream) == 0
            assert np.array_equal(idx.cpu().numpy(), ref), (M, N, ldy, wp is None)
        torch.cuda.synchronize()
        assert torch.count_nonzero(work[:65536]) == 0


@pytest.mark.parametrize("M,fused", [(1, True), (8, True), (3, True), (1, False), (8, False)])
def test_lm_head_greedy_workload(M, fused):
    """The greedy step on the LM head 151936 x 1024, with a workspace (the
    choice is the product launch's epilogue) and without (product, then a
    whole-row argmax): the logits within the product tolerance; the index
    bit-exact against the oracle's choice on the same fp32 logits; and
    against the fp64 logits, a value within the two tolerances of the true
    maximum (equal to it where the top two are further apart than that)."""
    bw, bx = weight_bits("lm_head", "w"), act_bits("lm_head", "x_m8")[:M]
    if M in (1, 8):
        bx = act_bits("lm_head", "x_m%d" % M)
    w = gpu_quant(bw)
    work = ws_for(fp4.OP_LM_HEAD_GREEDY, M, 1024, [151936]) if fused else None
    idx, logits = fp4.lm_head_greedy(to_gpu_bf16(bx), w, workspace=work)
    torch.cuda.synchronize()
    if fused:
        assert torch.count_nonzero(work[:65536]) == 0
    idx, lg = idx.cpu().numpy(), logits.cpu().numpy()
    p, s, g = oracle_quant("lm_head", "w")
    yr, l1 = oracle.gemv(bx, p, s, g, threads=THREADS)
    assert_within_tolerance(lg, yr, l1, "lm_head logits M=%d" % M)
    assert np.array_equal(idx, oracle.argmax_rows(lg))
    ref = oracle.argmax_rows(yr)
    for m in range(M):
        tol = 2e-3 * (l1[m, idx[m]] + l1[m, ref[m]])
        assert yr[m, idx[m]] >= yr[m, ref[m]] - tol
        second = np.partition(yr[m], -2)[-2]
        if yr[m, ref[m]] - second > 2e-3 * 2 * l1[m].max():
            assert idx[m] == ref[m]


# ------------------------------------------------------------- graph replay
def _graph_case():
    """Weights, inputs and outputs of the calls the bench replays from graphs."""
    ws = {name: gpu_quant(bf16_tensor(shape, 600 + i, 0.02, outlier_p=0.002, outlier_scale=20.0))
          for i, (name, shape) in enumerate([("g", (2048, 2048)), ("u", (2048, 2048)), ("d", (1000, 3072)),
                                              ("p1", (300, 1040)), ("p2", (1000, 1040)), ("lm", (20000, 1024))])}
    xs = {"x1": to_gpu_bf16(bf16_tensor((1, 2048), 71, 1.0)), "x8": to_gpu_bf16(bf16_tensor((8, 3072), 72, 1.0)),
          "xp": to_gpu_bf16(bf16_tensor((300, 1040), 73, 1.0)), "xl": to_gpu_bf16(bf16_tensor((1, 1024), 74, 1.0))}
    return ws, xs


def _graph_outs():
    return {"gu": torch.empty((1, 4096), dtype=torch.float32, device=dev()),
            "d8": torch.empty((8, 1000), dtype=torch.float32, device=dev()),
            "d8a": torch.empty((8, 1000), dtype=torch.float32, device=dev()),
            "pf": torch.empty((300, 1300), dtype=torch.float32, device=dev()),
            "lg": torch.empty((1, 20000), dtype=torch.float32, device=dev()),
            "ix": torch.empty((1,), dtype=torch.int32, device=dev())}


def _graph_step(ws, xs, o, work):
    fp4.gemv_multi(xs["x1"], [ws["g"], ws["u"]], [o["gu"][:, :2048], o["gu"][:, 2048:]], [4096, 4096])
    fp4.gemv(xs["x8"], ws["d"], out=o["d8"], workspace=work)
    fp4.gemv(xs["x8"], ws["d"], out=o["d8a"])          # no workspace: fill kernel + atomic adds
    fp4.gemm_prefill_multi(xs["xp"], [ws["p1"], ws["p2"]], [o["pf"][:, :300], o["pf"][:, 300:]], [1300, 1300],
                           workspace=work)
    fp4.lm_head_greedy(xs["xl"], ws["lm"], logits=o["lg"], out=o["ix"], workspace=work)


def _graph_work():
    need = max(fp4.workspace_bytes(fp4.OP_GEMV, 8, 3072, [1000]),
               fp4.workspace_bytes(fp4.OP_GEMM_PREFILL, 300, 1040, [300, 1000]),
               fp4.workspace_bytes(fp4.OP_LM_HEAD_GREEDY, 1, 1024, [20000]))
    return fp4.new_workspace(need, dev())


def test_graph_replays_match_eager_results():
    """The calls the bench replays from HIP graphs — the fused M = 1 product,
    the M = 8 matrix-core product with its K-chunk reduce (workspace) and
    with atomic adds (none), the fused prefill product with a K-split tail,
    and the greedy step folded into the LM-head launch, all sharing one
    workspace — captured once, replayed four times with eager work and
    synchronisations between the replays; every replay equals the eager
    results bit for bit (the atomic-add product: within the tolerance of the
    eager one, since its summation order is free)."""
    ws, xs = _graph_case()
    outs, work = _graph_outs(), _graph_work()
    _graph_step(ws, xs, outs, work)          # eager
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _graph_step(ws, xs, outs, work)
    torch.cuda.synchronize()
    scratch = _graph_outs()
    bd = bf16_tensor((1000, 3072), 602, 0.02, outlier_p=0.002, outlier_scale=20.0)
    p, s, gsc = oracle.quantize(bd)
    yr, l1 = oracle.gemv(bf16_tensor((8, 3072), 72, 1.0), p, s, gsc)
    for rep in range(4):
        for v in outs.values():
            v.fill_(float("nan") if v.dtype == torch.float32 else -1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            if k == "d8a":
                assert_within_tolerance(outs[k].cpu().numpy(), yr, l1, "atomic replay %d" % rep)
            else:
                assert torch.equal(outs[k], ref[k]), (rep, k)
        _graph_step(ws, xs, scratch, work)   # eager work between the replays
        torch.cuda.synchronize()
        for k in outs:
            if k != "d8a":
                assert torch.equal(scratch[k], ref[k]), (rep, k, "eager")
        assert torch.count_nonzero(work[:65536]) == 0


_FIRST_CALLS_UNDER_CAPTURE = r"""
import sys, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import test_gpu_parity as t
import bit_block_scaled_fp4_amd as fp4
t.fp4 = fp4
ws, xs = t._graph_case()
outs, work = t._graph_outs(), t._graph_work()
torch.cuda.synchronize()
side = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.stream(side):
    with torch.cuda.graph(g, stream=side):     # the process's first product calls
        t._graph_step(ws, xs, outs, work)
torch.cuda.synchronize()
g.replay(); g.replay()
torch.cuda.synchronize()
eager = t._graph_outs()
t._graph_step(ws, xs, eager, work)
torch.cuda.synchronize()
for k in outs:
    if k != "d8a":
        assert torch.equal(outs[k], eager[k]), k
print("first calls under capture ok", flush=True)
"""


def test_first_calls_under_graph_capture():
    """A process whose first product, prefill and greedy calls are made while
    the stream is captured into a graph (the library allocates nothing and
    sets up nothing on the stream on a first call); the replays equal eager
    results. Runs in a fresh process, since this one has made such calls."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALLS_UNDER_CAPTURE, root], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and "capture ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


def test_two_streams_at_once():
    """The 27B down projection at M = 8 (matrix cores, 17 K chunks) on one
    stream and the LM-head greedy step (M = 1, choice in the product launch)
    on another, both default priority, issued back to back three times before
    one synchronisation: first each with its own workspace, then both without
    (atomic adds; whole-row argmax). Every result against the oracle: the
    products within the tolerance, the indices equal to the oracle's choice
    on the GPU's logits."""
    print("two streams", flush=True)
    wd = gpu_quant(weight_bits("dense27b_layer", "down"))
    wl = gpu_quant(weight_bits("lm_head", "w"))
    bx8, bxl = act_bits("dense27b_smallm", "x_mid_m8"), act_bits("lm_head", "x_m1")
    x8, xl = to_gpu_bf16(bx8), to_gpu_bf16(bxl)
    wa = ws_for(fp4.OP_GEMV, 8, 17408, [5120])
    wb = ws_for(fp4.OP_LM_HEAD_GREEDY, 1, 1024, [151936])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    res = []
    for use_ws in (True, False):
        ys = [torch.full((8, 5120), float("nan"), device=dev()) for _ in range(3)]
        lgs = [torch.empty((1, 151936), device=dev()) for _ in range(3)]
        ixs = [torch.full((1,), -1, dtype=torch.int32, device=dev()) for _ in range(3)]
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        for r in range(3):
            with torch.cuda.stream(s1):
                fp4.gemv(x8, wd, out=ys[r], workspace=wa if use_ws else None)
            with torch.cuda.stream(s2):
                fp4.lm_head_greedy(xl, wl, logits=lgs[r], out=ixs[r], workspace=wb if use_ws else None)
        torch.cuda.synchronize()
        res.append((use_ws, ys, lgs, ixs))
    pd, sd, gd = oracle_quant("dense27b_layer", "down")
    yr, l1 = oracle.gemv(bx8, pd, sd, gd, threads=THREADS)
    pl, sl, gl = oracle_quant("lm_head", "w")
    yl, ll1 = oracle.gemv(bxl, pl, sl, gl, threads=THREADS)
    for use_ws, ys, lgs, ixs in res:
        for r in range(3):
            assert_within_tolerance(ys[r].cpu().numpy(), yr, l1, "down M=8 ws=%s rep %d" % (use_ws, r))
            lg = lgs[r].cpu().numpy()
            assert_within_tolerance(lg, yl, ll1, "lm head ws=%s rep %d" % (use_ws, r))
            assert np.array_equal(ixs[r].cpu().numpy(), oracle.argmax_rows(lg)), (use_ws, r)
        if use_ws:
            assert all(torch.equal(ys[0], y) for y in ys)
    assert torch.count_nonzero(wa[:65536]) == 0 and torch.count_nonzero(wb[:65536]) == 0


# --------------------------------------------- fused neighbours: RMSNorm, SwiGLU
def gain_bits(K, seed):
    return norm_gain(K, seed)


# Bound of the normalised product: the product bound on the normalised rows,
# plus one bf16 rounding (2^-9 relative) of each normalised input and the
# fp32 norm's own error (below 1e-4 relative for K <= 2^20), all relative to
# sum_k |w * xn|.
RMS_TOL = 2e-3 + 2.0 ** -9 + 1e-4


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_rmsnorm_then_qkv(M):
    """Q, K and V of the Qwen3-0.6B-shaped layer 1 (2048, 1024, 1024 x 1024)
    in one call on the RMS-normalised rows (gain ~ 1 + N(0, 0.1), eps 1e-6,
    rows ~ N(0, 3)): M <= 2 inside the product's launch, M = 4 and 8 through
    the norm kernel and a workspace. Against the oracle's fp64 norm and
    product within RMS_TOL * sum|w * xn|; the plain product of the raw rows
    does not meet that bound (the norm is really applied)."""
    wl, K = "qwen3_0p6b_decode", 1024
    names, Ns = ("q", "k", "v"), (2048, 1024, 1024)
    ws = [gpu_quant(weight_bits(wl, "L1.%s" % t)) for t in names]
    bx = bf16_tensor((M, K), 7100 + M, 3.0)
    gb = gain_bits(K, 55)
    x, gain = to_gpu_bf16(bx), to_gpu_bf16(gb)
    qkv = torch.full((M, 4096), float("nan"), device=dev())
    outs = [qkv, qkv[:, 2048:], qkv[:, 3072:]]
    need = fp4.workspace_bytes(fp4.OP_GEMV_RMSNORM, M, K, list(Ns))
    assert (need == 0) == (M <= 2)
    work = fp4.new_workspace(need, dev()) if need else None
    if need:
        with pytest.raises(fp4.Fp4Error):
            fp4.gemv_multi_rmsnorm(x, gain, 1e-6, ws, outs, [4096] * 3)
    fp4.gemv_multi_rmsnorm(x, gain, 1e-6, ws, outs, [4096] * 3, workspace=work)
    raw = fp4.gemv(x, ws[0])
    torch.cuda.synchronize()
    xn = oracle.rmsnorm(bx, gb, 1e-6)
    off = 0
    for i, (t, N) in enumerate(zip(names, Ns)):
        p, s, g = oracle_quant(wl, "L1.%s" % t)
        yr, l1 = oracle.gemv_f64(xn, p, s, g)
        ok, worst = oracle.tolerance_ok(qkv[:, off:off + N].cpu().numpy().astype(np.float64), yr, l1, RMS_TOL)
        assert ok, "%s M=%d worst %.3g" % (t, M, worst)
        if i == 0:
            assert not oracle.tolerance_ok(raw.cpu().numpy().astype(np.float64), yr, l1, RMS_TOL)[0]
        off += N


def swiglu_bound(g, u, l1g, l1u, h):
    """|h_gpu - silu(g) u| bound from the product bounds on g and u
    (|dg| <= 2e-3 l1g, |du| <= 2e-3 l1u), silu's slope (at most 1.1), one
    bf16 rounding of the result and fp32 evaluation (2^-8 of |h|)."""
    sg = np.abs(oracle.swiglu(g, np.ones_like(g)))
    prod = 1.1 * 2e-3 * l1g * (np.abs(u) + 2e-3 * l1u) + sg * 2e-3 * l1u
    return prod * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(h) + 1e-30


@pytest.mark.parametrize("case,M", [("27b", 1), ("27b", 2), ("27b", 8), ("qwen", 1), ("qwen", 4)])
def test_gemv_swiglu(case, M):
    """h = bf16(silu(gate) * up) for the 27B-class gate/up (17408 x 5120) at
    M = 1, 2 (one vector-ALU launch) and 8 (matrix-core product into the
    workspace, then the elementwise kernel), and the Qwen3-0.6B-shaped layer
    1 (3072 x 1024) at M = 1 and 4; against the oracle's fp64 products and
    silu within swiglu_bound; the operands swapped do not meet it."""
    if case == "27b":
        wl, pre, K = "dense27b_layer", "", 5120
        bx = act_bits(wl, "x_in") if M == 1 else act_bits("dense27b_smallm", "x_in_m%d" % M)
    else:
        wl, pre, K = "qwen3_0p6b_decode", "L1.", 1024
        bx = bf16_tensor((M, K), 7300 + M, 1.0)
    print("swiglu", case, M, flush=True)
    wg, wu = gpu_quant(weight_bits(wl, pre + "gate")), gpu_quant(weight_bits(wl, pre + "up"))
    N = wg.N
    need = fp4.workspace_bytes(fp4.OP_GEMV_SWIGLU, M, K, [N])
    work = fp4.new_workspace(need, dev()) if need else None
    h = fp4.gemv_swiglu(to_gpu_bf16(bx), wg, wu, workspace=work)
    torch.cuda.synchronize()
    hg = bf16_to_float32(h.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    pg, sg, gg = oracle_quant(wl, pre + "gate")
    pu, su, gu = oracle_quant(wl, pre + "up")
    g, l1g = oracle.gemv(bx, pg, sg, gg, threads=THREADS)
    u, l1u = oracle.gemv(bx, pu, su, gu, threads=THREADS)
    href = oracle.swiglu(g, u)
    bound = swiglu_bound(g, u, l1g, l1u, href)
    err = np.abs(hg - href)
    assert np.all(err <= bound), "worst %.3g" % float((err / bound).max())
    assert not np.all(np.abs(hg - oracle.swiglu(u, g)) <= swiglu_bound(u, g, l1u, l1g, oracle.swiglu(u, g)))


def test_neighbours_long_k_two_rows():
    """The fused neighbours at M = 2 over 8 or more K chunks, where the
    vector-ALU launch runs one row group of 8 waves per projection (SwiGLU:
    gate and up together, 16 waves): SwiGLU at K = 9216 (9 chunks, 136 rows)
    within swiglu_bound, and RMSNorm before two projections (200 and 64 rows)
    at K = 8192 within RMS_TOL * sum|w * xn|."""
    M = 2
    K = 9216
    bg, bu = (bf16_tensor((136, K), s, 0.03, outlier_p=0.002, outlier_scale=20.0) for s in (401, 402))
    bx = bf16_tensor((M, K), 403, 1.0)
    wg, wu = gpu_quant(bg), gpu_quant(bu)
    need = fp4.workspace_bytes(fp4.OP_GEMV_SWIGLU, M, K, [136])
    h = fp4.gemv_swiglu(to_gpu_bf16(bx), wg, wu, workspace=fp4.new_workspace(need, dev()) if need else None)
    torch.cuda.synchronize()
    hg = bf16_to_float32(h.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    g, l1g = oracle.gemv(bx, *oracle.quantize(bg), threads=THREADS)
    u, l1u = oracle.gemv(bx, *oracle.quantize(bu), threads=THREADS)
    href = oracle.swiglu(g, u)
    err = np.abs(hg - href)
    bound = swiglu_bound(g, u, l1g, l1u, href)
    assert np.all(err <= bound), "swiglu worst %.3g" % float((err / bound).max())

    K = 8192
    Ns = (200, 64)
    bws = [bf16_tensor((N, K), 410 + N, 0.03, outlier_p=0.002, outlier_scale=20.0) for N in Ns]
    ws = [gpu_quant(b) for b in bws]
    bx = bf16_tensor((M, K), 411, 3.0)
    gb = gain_bits(K, 56)
    outs = [torch.full((M, N), float("nan"), device=dev()) for N in Ns]
    need = fp4.workspace_bytes(fp4.OP_GEMV_RMSNORM, M, K, list(Ns))
    fp4.gemv_multi_rmsnorm(to_gpu_bf16(bx), to_gpu_bf16(gb), 1e-6, ws, outs, list(Ns),
                           workspace=fp4.new_workspace(need, dev()) if need else None)
    torch.cuda.synchronize()
    xn = oracle.rmsnorm(bx, gb, 1e-6)
    for b, o in zip(bws, outs):
        yr, l1 = oracle.gemv_f64(xn, *oracle.quantize(b))
        ok, worst = oracle.tolerance_ok(o.cpu().numpy().astype(np.float64), yr, l1, RMS_TOL)
        assert ok, "rmsnorm worst %.3g" % worst


# ------------------------------------------------------------------- MXFP4
_mx_cache = {}


def mx_oracle_quant(wl, name):
    key = (wl, name)
    if key not in _mx_cache:
        _mx_cache[key] = oracle.mx_quantize(weight_bits(wl, name))
    return _mx_cache[key]


def mx_edge_tensors():
    from test_oracle_pins import load_mx_example
    rng = np.random.default_rng(61)
    out = {"worked_example": load_mx_example()[0]}
    out["zeros"] = np.zeros((9, 64), np.uint16)
    out["ragged_13x1056"] = bf16_tensor((13, 1056), 62, 0.02, outlier_p=0.01, outlier_scale=20)
    out["tiny"] = float32_to_bf16_bits(rng.normal(0, 1e-30, (16, 64)).astype(np.float32))
    out["huge"] = float32_to_bf16_bits(rng.normal(0, 1e30, (16, 64)).astype(np.float32))
    wide = rng.normal(0, 1, (32, 256)) * np.exp(rng.uniform(-40, 40, (32, 256)))
    out["wide_dynamic_range"] = float32_to_bf16_bits(wide.astype(np.float32))
    return out


def check_mx_bytes(bits, what):
    p, s = oracle.mx_quantize(bits)
    w = fp4.quantize_mx(to_gpu_bf16(bits), "mx_rowmajor")
    wt = fp4.quantize_mx(to_gpu_bf16(bits), "mx_tiled")
    torch.cuda.synchronize()
    gp, gs = gpu_u8(w.packed).reshape(p.shape), gpu_u8(w.scales).reshape(s.shape)
    assert np.array_equal(gs, s), (what, np.flatnonzero(gs != s)[:8])
    assert np.array_equal(gp, p), (what, np.flatnonzero(gp != p)[:8])
    assert np.array_equal(gpu_u8(wt.packed), oracle.mx_tile(p, s)), what
    return p, s


@pytest.mark.parametrize("name", list(mx_edge_tensors().keys()))
def test_mx_quantize_bit_exact_edge_cases(name):
    check_mx_bytes(mx_edge_tensors()[name], name)


@pytest.mark.parametrize("wl,t", [("dense27b_layer", "gate"), ("dense27b_layer", "down"), ("lm_head", "w")])
def test_mx_quantize_bit_exact_workloads(wl, t):
    print("mx quantize", wl, t, flush=True)
    bits = weight_bits(wl, t)
    p, s = mx_oracle_quant(wl, t)
    w = fp4.quantize_mx(to_gpu_bf16(bits), "mx_rowmajor")
    wt = fp4.quantize_mx(to_gpu_bf16(bits), "mx_tiled")
    torch.cuda.synchronize()
    assert np.array_equal(gpu_u8(w.scales).reshape(s.shape), s)
    assert np.array_equal(gpu_u8(w.packed).reshape(p.shape), p)
    assert np.array_equal(gpu_u8(wt.packed), oracle.mx_tile(p, s))


@pytest.mark.parametrize("N,K,M", [(8, 32, 1), (13, 1056, 1), (40, 2080, 3), (333, 3072, 5), (1000, 1024, 9),
                                   (77, 17408 + 32, 2)])
def test_mx_gemv_small_shapes(N, K, M):
    bw = bf16_tensor((N, K), 6000 + N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 6100 + M, 1.0)
    w = fp4.quantize_mx(to_gpu_bf16(bw), "mx_tiled")
    y = fp4.gemv_mx(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s = oracle.mx_quantize(bw)
    yr, l1 = oracle.mx_gemv(bx, p, s)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "mx gemv %d %d %d" % (N, K, M))


@pytest.mark.parametrize("wl,t,xname", [("dense27b_layer", "gate", "x_in"), ("dense27b_layer", "down", "x_mid"),
                                        ("lm_head", "w", "x_m1"), ("lm_head", "w", "x_m8")])
def test_mx_gemv_workloads(wl, t, xname):
    """The 27B-class layer's projections at M = 1 and the LM head at M = 1
    and 8, MXFP4-quantised from the same bf16 weights."""
    print("mx gemv", wl, t, xname, flush=True)
    bx = act_bits(wl, xname)
    w = fp4.quantize_mx(to_gpu_bf16(weight_bits(wl, t)), "mx_tiled")
    y = fp4.gemv_mx(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s = mx_oracle_quant(wl, t)
    yr, l1 = oracle.mx_gemv(bx, p, s)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "mx %s %s" % (t, xname))


@pytest.mark.parametrize("M,N,K", [(1, 8, 32), (37, 300, 1056), (200, 129, 2048), (300, 1000, 5120),
                                   (257, 16400, 1056)])
def test_mx_prefill_small_shapes(M, N, K):
    print("mx prefill", M, N, K, flush=True)
    bw = bf16_tensor((N, K), 6200 + M + N + K, 0.02, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 6300 + M, 1.0)
    w = fp4.quantize_mx(to_gpu_bf16(bw), "mx_tiled")
    y = fp4.gemm_prefill_mx(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    p, s = oracle.mx_quantize(bw)
    yr, l1 = oracle.mx_gemv(bx, p, s)
    assert_within_tolerance(y.cpu().numpy(), yr, l1, "mx prefill %d %d %d" % (M, N, K))


@pytest.mark.parametrize("name", list(mx_edge_tensors().keys()))
def test_mx_products_on_edge_tensors(name):
    """The MXFP4 decode product and prefill on the edge tensors (zeros, tiny
    ~1e-30 and huge ~1e30 weights, a wide dynamic range, a ragged shape, the
    worked example): the prefill decodes E8M0-scaled codes in one conversion
    whose scale operand carries the shared exponent, far from 2^0 here. Both
    within the tolerance of the oracle (products of zero rows exactly 0)."""
    bw = mx_edge_tensors()[name]
    N, K = bw.shape
    print("mx edge products", name, N, K, flush=True)
    w = fp4.quantize_mx(to_gpu_bf16(bw), "mx_tiled")
    p, s = oracle.mx_quantize(bw)
    for M in (1, 37):
        bx = bf16_tensor((M, K), 6400 + M + N, 1.0)
        x = to_gpu_bf16(bx)
        yg = fp4.gemv_mx(x, w)
        yp = fp4.gemm_prefill_mx(x, w)
        torch.cuda.synchronize()
        yr, l1 = oracle.mx_gemv(bx, p, s)
        assert_within_tolerance(yg.cpu().numpy(), yr, l1, "mx edge gemv %s M=%d" % (name, M))
        assert_within_tolerance(yp.cpu().numpy(), yr, l1, "mx edge prefill %s M=%d" % (name, M))


def test_mx_prefill_full_size_sampled_rows():
    """2048 tokens x the 27B-class gate projection 17408 x 5120 in MXFP4,
    checked on 8 sampled token rows (all 17408 outputs each)."""
    bx = act_bits("prefill", "x")
    w = fp4.quantize_mx(to_gpu_bf16(weight_bits("dense27b_layer", "gate")), "mx_tiled")
    y = fp4.gemm_prefill_mx(to_gpu_bf16(bx), w)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 1000, 1791, 1792, 2047]
    p, s = mx_oracle_quant("dense27b_layer", "gate")
    yr, l1 = oracle.mx_gemv(bx[rows], p, s)
    assert_within_tolerance(y[rows].cpu().numpy(), yr, l1, "mx prefill full size")


# ------------------------------------------------ both operands MXFP4 (R28)
def check_mx_a4(y_gpu, y_ref, l1, what):
    """The block-scaled FP4 product against the oracle's fp64 product of the
    two dequantised operands: every product is exact and the sums are fp32,
    so the bar is 1e-4 of sum |a*w| (twenty times tighter than the products
    with bf16 activations)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), what
    ok, worst = oracle.tolerance_ok(y_gpu, y_ref, l1, rel=1e-4)
    assert ok, "%s: |y_gpu - y_ref| exceeds 1e-4*sum|a*w| (worst ratio %.3g)" % (what, worst)


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (37, 300, 1152), (256, 128, 128), (300, 520, 2048),
                                   (513, 1000, 5120)])
def test_mx_a4_small_shapes(M, N, K):
    """Both operands MXFP4 on the block-scaled FP4 matrix cores: the
    activations quantised on the GPU bit-exact against the oracle's MXFP4
    rule, and the product within 1e-4 of sum |a*w|. Shapes: one row; ragged
    rows and columns over several 256 x 128 tiles (a last row tile of one
    row, last column tiles of 44 and 104 columns, a ragged last weight row
    group); 1, 9, 16 and 40 K steps, K a whole or a partial tile chunk."""
    print("mx a4", M, N, K, flush=True)
    bw = bf16_tensor((N, K), 9 * N + K, 0.03, outlier_p=0.002, outlier_scale=20.0)
    bx = bf16_tensor((M, K), 13 * M + K, 1.0, outlier_p=0.002, outlier_scale=20.0)
    w = fp4.quantize_mx(to_gpu_bf16(bw), "mx_tiled")
    xq = fp4.quantize_mx(to_gpu_bf16(bx), "mx_act")
    y = fp4.gemm_mx_a4(xq, w)
    torch.cuda.synchronize()
    xp, xs = oracle.mx_quantize(bx)
    assert np.array_equal(xq.packed.cpu().numpy().reshape(M, K // 2), xp)
    # activation layout: the scales of each 128-column step, rows consecutive
    xs_gpu = xq.scales.cpu().numpy().reshape(K // 128, M, 4).transpose(1, 0, 2).reshape(M, K // 32)
    assert np.array_equal(xs_gpu, xs)
    wp, ws = oracle.mx_quantize(bw)
    yr, l1 = oracle.mx_a4_product(xp, xs, wp, ws)
    check_mx_a4(y.cpu().numpy(), yr, l1, "mx a4 %dx%dx%d" % (M, N, K))


def test_mx_a4_full_size_sampled_rows():
    """2048 tokens x the 27B-class gate projection 17408 x 5120, both operands
    MXFP4, checked on 8 sampled token rows (all 17408 outputs each)."""
    bx = act_bits("prefill", "x")
    w = fp4.quantize_mx(to_gpu_bf16(weight_bits("dense27b_layer", "gate")), "mx_tiled")
    xq = fp4.quantize_mx(to_gpu_bf16(bx), "mx_act")
    y = fp4.gemm_mx_a4(xq, w)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 1000, 1791, 1792, 2047]
    p, s = mx_oracle_quant("dense27b_layer", "gate")
    xp, xs = oracle.mx_quantize(bx[rows])
    yr, l1 = oracle.mx_a4_product(xp, xs, p, s)
    check_mx_a4(y[rows].cpu().numpy(), yr, l1, "mx a4 full size")


def test_mx_a4_8192_rows_sampled():
    """8192 tokens x the gate projection: 2176 tiles, so each workgroup of the
    persistent grid walks 8 or 9 of them; 6 sampled rows (first and last
    rows, tile and band edges), all 17408 outputs each."""
    print("mx a4 8192 rows", flush=True)
    bx = bf16_tensor((8192, 5120), 8192 * 7 + 5, 1.0, outlier_p=0.001, outlier_scale=20.0)
    w = fp4.quantize_mx(to_gpu_bf16(weight_bits("dense27b_layer", "gate")), "mx_tiled")
    xq = fp4.quantize_mx(to_gpu_bf16(bx), "mx_act")
    y = fp4.gemm_mx_a4(xq, w)
    torch.cuda.synchronize()
    rows = [0, 255, 256, 4095, 8064, 8191]
    p, s = mx_oracle_quant("dense27b_layer", "gate")
    xp, xs = oracle.mx_quantize(bx[rows])
    yr, l1 = oracle.mx_a4_product(xp, xs, p, s)
    check_mx_a4(y[rows].cpu().numpy(), yr, l1, "mx a4 8192 rows")
