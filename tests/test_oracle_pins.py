"""Pins for the CPU oracle: each check compares it with something other than
itself (the format's bit-field definition, torch's float8_e4m3fn, brute-force
search, exact rational arithmetic, numpy float64 matmul, a hand-worked
example), chosen so that a dropped term, a wrong sign or index, a swapped
nibble or a transposed operand fails at least one of them."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_tensor, bf16_to_float32, float32_to_bf16_bits, tensor_bits, workload, x_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- E2M1 values
def minifloat_value(code, ebits, mbits, bias):
    """Value of a sign/exponent/mantissa minifloat from its bit fields."""
    s = code >> (ebits + mbits)
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if s else v


def test_e2m1_values_match_bit_fields():
    # E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit.
    for c in range(16):
        assert oracle.e2m1_value(c) == float(minifloat_value(c, 2, 1, 1))
        assert np.signbit(oracle.e2m1_value(c)) == bool(c & 8)
    mags = sorted({abs(oracle.e2m1_value(c)) for c in range(16)})
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ----------------------------------------------------------------- E4M3 decode
def test_e4m3_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c] and np.signbit(v) == np.signbit(ref[c]), (c, v, ref[c])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_decode_matches_bit_fields():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_value(c) == float(minifloat_value(c, 4, 3, 7))


# ----------------------------------------------------------------- E4M3 encode
def _neighbourhood(values, ulps):
    v = np.asarray(values, dtype=np.float32)
    bits = v.view(np.int32)
    out = [(bits + d).view(np.float32) for d in range(-ulps, ulps + 1)]
    return np.concatenate(out)


def test_e4m3_encode_matches_torch_rne():
    finite = np.array([oracle.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
    mids = (finite[:-1] + finite[1:]) / 2
    pts = np.concatenate([_neighbourhood(finite[1:].astype(np.float32), 3),
                          _neighbourhood(mids.astype(np.float32), 3),
                          np.array([0.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 448.0, 460.0, 463.99], np.float32)])
    rng = np.random.default_rng(0)
    rnd = np.exp(rng.uniform(np.log(1e-5), np.log(463.0), 2_000_000)).astype(np.float32)
    s = np.concatenate([pts, rnd])
    s = s[(s >= 0) & (s < 464.0)]
    ours = oracle.e4m3_encode_array(s)
    ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def test_e4m3_encode_saturates_and_round_trips():
    big = np.array([448.0, 449.0, 464.0, 470.0, 1e6, 3e38, np.inf], np.float32)
    assert np.all(oracle.e4m3_encode_array(big) == 0x7E)
    for c in range(0x7F):
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c


# ----------------------------------------------------------------- E2M1 encode
def e2m1_bruteforce(v):
    """Nearest of the 16 codes by exhaustive search; ties to the code whose
    mantissa bit is 0; |v| > 6 saturates; sign from the sign bit of v."""
    mags = np.array([float(minifloat_value(c, 2, 1, 1)) for c in range(8)])
    a = np.abs(v.astype(np.float64))[:, None]
    d = np.abs(a - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def test_e2m1_encode_matches_bruteforce():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = ((mags[:-1].astype(np.float64) + mags[1:]) / 2).astype(np.float32)
    pts = np.concatenate([_neighbourhood(mags[1:], 8), _neighbourhood(mids, 8), [0.0, 1e-30, 6.5, 7.0, 100.0]])
    pts = np.concatenate([pts, -pts, np.float32([-0.0])]).astype(np.float32)
    rng = np.random.default_rng(1)
    rnd = rng.uniform(-8, 8, 1_000_000).astype(np.float32)
    v = np.concatenate([pts, rnd])
    assert np.array_equal(oracle.e2m1_encode_array(v), e2m1_bruteforce(v))


# ------------------------------------------------------------------ quantiser
def load_worked_example():
    rows, packed, scales, gscale = [], [], [], None
    with open(os.path.join(GOLDEN, "quant_worked_example.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "gscale":
                gscale = float(vals[0])
            elif key == "row":
                rows.append([float(v) for v in vals])
            elif key == "packed":
                packed.append([int(v, 16) for v in vals])
            elif key == "scales":
                scales.append([int(v, 16) for v in vals])
    W = np.array(rows, dtype=np.float32)
    Wb = float32_to_bf16_bits(W)
    assert np.array_equal(bf16_to_float32(Wb), W) and np.array_equal(np.signbit(bf16_to_float32(Wb)), np.signbit(W))
    return Wb, np.array(packed, np.uint8), np.array(scales, np.uint8), np.float32(gscale)


def test_quantize_worked_example():
    Wb, packed, scales, g = load_worked_example()
    p, s, gs = oracle.quantize(Wb)
    assert gs == g
    assert np.array_equal(s, scales), (s, scales)
    assert np.array_equal(p, packed), (p, packed)


def check_invariants(Wb, p, s, g):
    W = bf16_to_float32(Wb).astype(np.float64)
    N, K = W.shape
    amax = np.abs(W).max()
    assert g == np.float32(np.float32(amax) / np.float32(2688.0))
    assert s.max() <= 0x7E and not np.any(s & 0x80)
    blk = np.abs(W).reshape(N, K // 16, 16).max(axis=2)
    n0, b0 = np.unravel_index(np.argmax(blk), blk.shape)
    assert s[n0, b0] == 0x7E
    D = oracle.dequant(p, s, g)
    sdec = np.array([oracle.e4m3_value(c) for c in range(256)])[s]            # [N][K/16]
    d = np.repeat(sdec * float(g), 16, axis=1)
    normal = np.repeat(s >= 0x08, 16, axis=1)
    assert np.all(np.abs(W - D)[normal] <= d[normal] * (1 + 2.0 ** -20))
    # the largest element of each normal-scale block decodes to +-6 * s_dec * gscale
    idx = np.argmax(np.abs(W).reshape(N, K // 16, 16), axis=2)
    q = np.stack([p & 15, p >> 4], axis=2).reshape(N, K // 16, 16)
    top = np.take_along_axis(q, idx[..., None], axis=2)[..., 0]
    Wtop = np.take_along_axis(W.reshape(N, K // 16, 16), idx[..., None], axis=2)[..., 0]
    sel = (s >= 0x08) & (Wtop != 0)
    assert np.all((top[sel] & 7) == 7)
    assert np.all(((top[sel] & 8) != 0) == (Wtop[sel] < 0))


@pytest.mark.parametrize("name,tname,rows", [("gemv_1024", "w", None), ("dense27b_layer", "down", 256),
                                             ("lm_head", "w", 512), ("qwen3_0p6b_decode", "L1.q", None)])
def test_quantize_invariants_on_workloads(name, tname, rows):
    W = tensor_bits(workload(name).tensor(tname))
    if rows:
        W = W[:rows]
    p, s, g = oracle.quantize(W)
    check_invariants(W, p, s, g)


def test_quantize_degenerate_cases():
    z = np.zeros((4, 32), np.uint16)
    p, s, g = oracle.quantize(z)
    assert g == 0 and not p.any() and not s.any()
    one = np.zeros((2, 32), np.float32)
    one[1, 20] = -0.75
    p, s, g = oracle.quantize(float32_to_bf16_bits(one))
    assert g == np.float32(0.75) / np.float32(2688)
    assert list(s.ravel()) == [0, 0, 0, 0x7E]
    assert p[1, 10] == 0x0F and p[1].sum() == 0x0F        # k=20 is the low nibble of byte 10, code -6
    const = np.full((1, 16), 0.3, np.float32)
    p, s, g = oracle.quantize(float32_to_bf16_bits(const))
    assert s[0, 0] == 0x7E and np.all(p == 0x77)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 24), np.uint16))


# -------------------------------------------------------------------- product
def dequant_from_bits(p, s, g):
    """Dequantised weights built independently of the oracle: E2M1 from its
    bit fields, E4M3 through torch.float8_e4m3fn."""
    e2 = np.array([float(minifloat_value(c, 2, 1, 1)) for c in range(16)])
    e4 = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e4m3fn).double().numpy()
    q = np.stack([p & 15, p >> 4], axis=2).reshape(p.shape[0], -1)
    return e2[q] * np.repeat(e4, 16, axis=1) * float(g)


def test_gemv_matches_numpy_on_tiny_matrices():
    rng = np.random.default_rng(3)
    for N, K, M in [(1, 16, 1), (3, 32, 2), (7, 64, 3), (64, 48, 4), (5, 1024 + 16, 2)]:
        W = float32_to_bf16_bits(rng.normal(0, 0.05, (N, K)).astype(np.float32))
        x = float32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
        p, s, g = oracle.quantize(W)
        D = dequant_from_bits(p, s, g)
        xf = bf16_to_float32(x).astype(np.float64)
        y, l1 = oracle.gemv(x, p, s, g)
        ref = xf @ D.T
        assert np.allclose(y, ref, rtol=1e-13, atol=1e-15 * np.abs(D).sum())
        assert np.allclose(l1, np.abs(xf) @ np.abs(D).T, rtol=1e-13)
        assert not np.allclose(y, (xf[:, ::-1] @ D.T) if K > 16 else y + 1)


def test_gemv_exact_against_rationals():
    """Worked example weights with power-of-two x: every product and sum is a
    short binary fraction, so the fp64 result must equal exact rational
    arithmetic over the bit-field decodes."""
    Wb, packed, scales, g = load_worked_example()
    rng = np.random.default_rng(4)
    x = (2.0 ** rng.integers(-3, 4, (3, 32))) * rng.choice([-1, 1], (3, 32))
    xb = float32_to_bf16_bits(x.astype(np.float32))
    y, _ = oracle.gemv(xb, packed, scales, g)
    e2 = [minifloat_value(c, 2, 1, 1) for c in range(16)]
    e4 = [minifloat_value(c, 4, 3, 7) for c in range(0x7F)]
    for m in range(3):
        for n in range(2):
            acc = Fraction(0)
            for k in range(32):
                q = packed[n, k // 2] >> (4 * (k % 2)) & 15
                acc += e2[q] * e4[scales[n, k // 16]] * Fraction(float(g)) * Fraction(float(x[m, k]))
            assert y[m, n] == float(acc)


def test_gemv_one_hot_selects_a_column():
    W = tensor_bits(workload("gemv_1024").tensor("w"))[:64]
    p, s, g = oracle.quantize(W)
    D = dequant_from_bits(p, s, g)
    for k in [0, 1, 15, 16, 17, 511, 1023]:
        x = np.zeros((1, 1024), np.float32)
        x[0, k] = 1.0
        y, _ = oracle.gemv(float32_to_bf16_bits(x), p, s, g)
        assert np.array_equal(y[0], D[:, k])


def test_gemv_threads_do_not_change_results():
    W = tensor_bits(workload("gemv_1024").tensor("w"))
    x = x_bits(workload("gemv_1024").x("x"))
    p, s, g = oracle.quantize(W)
    y1, l1 = oracle.gemv(x, p, s, g, threads=1)
    y8, l8 = oracle.gemv(x, p, s, g, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(l1, l8)


def test_tolerance_helper():
    ok, r = oracle.tolerance_ok(np.array([1.0, 2.0]), np.array([1.0, 2.001]), np.array([1.0, 1.0]))
    assert ok and abs(r - 0.5) < 1e-9
    ok, r = oracle.tolerance_ok(np.array([1.0]), np.array([1.01]), np.array([1.0]))
    assert not ok


# ---------------------------------------------------------------- tiled layout
def test_tile_matches_reshape_formulation():
    rng = np.random.default_rng(5)
    for N, K in [(16, 2048), (24, 1024), (8, 3072)]:
        p = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = rng.integers(0, 256, (N, K // 16), dtype=np.uint8)
        t = oracle.tile(p, s).reshape(-1, 4608)
        G, C = N // 8, K // 1024
        # codes: [g][r][c][l][i] -> [g][c][r][l][i]; scales: row r = 2i + h,
        # [g][i][h][c][l][j] -> [g][c][h][l][i][j]
        ref_p = p.reshape(G, 8, C, 32, 16).transpose(0, 2, 1, 3, 4).reshape(G * C, 4096)
        ref_s = s.reshape(G, 4, 2, C, 32, 2).transpose(0, 3, 2, 4, 1, 5).reshape(G * C, 512)
        assert np.array_equal(t[:, :4096], ref_p) and np.array_equal(t[:, 4096:], ref_s)


def test_tile_pads_ragged_shapes_with_zeros():
    N, K = 11, 1024 + 48
    p = np.arange(N * K // 2, dtype=np.int64).astype(np.uint8).reshape(N, K // 2) | 1
    s = np.full((N, K // 16), 0x33, np.uint8)
    t = oracle.tile(p, s).reshape(-1, 4608)
    assert t.shape == (2 * 2, 4608)
    pt, st = t[:, :4096].ravel(), t[:, 4096:].ravel()
    assert np.count_nonzero(pt) == N * K // 2 and np.count_nonzero(st) == N * K // 16
    assert np.array_equal(np.sort(pt[pt != 0]), np.sort(p.ravel()))


# ------------------------------------------------------------- greedy choice
# Greedy decoding picks the largest logit of the last position (page "1. The
# big picture", steps 4 and 5). The oracle's rule: the first index of the
# largest value, NaN above every number, -0 equal to +0.
def test_argmax_rows_matches_python_max_with_ties():
    rng = np.random.default_rng(123)
    for N in (1, 2, 7, 64, 1000):
        y = rng.integers(-3, 4, size=(5, N)).astype(np.float32)   # many equal values
        got = oracle.argmax_rows(y)
        for m in range(5):
            row = [float(v) for v in y[m]]
            # the built-in max returns the first maximal item it meets
            assert got[m] == max(range(N), key=lambda n: row[n])


def test_argmax_rows_matches_numpy_with_nan_inf_and_signed_zero():
    rng = np.random.default_rng(7)
    for dt in (np.float64, np.float32):
        y = rng.standard_normal((6, 300)).astype(dt)
        y[1, 17] = np.nan
        y[1, 200] = np.nan            # the first NaN wins
        y[2, :] = 0.0
        y[2, 0] = -0.0                # -0 ties with +0: index 0
        y[3, :] = -np.inf
        y[3, 9] = -1e30               # the only finite value
        y[4, 250] = np.inf
        y[5, :] = y[5, 123]           # a constant row: index 0
        got = oracle.argmax_rows(y)
        assert np.array_equal(got, np.argmax(y, axis=1).astype(np.int32))
        assert got.tolist() == [int(np.argmax(y[0])), 17, 0, 9, 250, 0]


def test_argmax_rows_decides_in_the_given_precision():
    y64 = np.array([[1.0, 1.0 + 2.0 ** -40, 0.5]])
    assert oracle.argmax_rows(y64).tolist() == [1]
    # both round to 1.0 in fp32: the first one wins
    assert oracle.argmax_rows(y64.astype(np.float32)).tolist() == [0]


# ------------------------------------------------------- FP8-sourced weights
# A checkpoint released in FP8 (imp README: the quantiser builds NVFP4 weights
# from BF16 or FP8 releases) holds E4M3 codes and a dequantisation scale; the
# element values E4M3(code) * scale, rounded once to fp32, go through the same
# quantisation rule. The E4M3 decode below is torch's, not the oracle's.
def fp8_codes(shape, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E          # no NaN codes (outside the domain)
    c.flat[::97] = 0                       # some zeros
    c.flat[5::131] = 0x80                  # and negative zeros
    return c


def torch_e4m3_values(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_quantize_fp8_with_power_of_two_scale_equals_bf16_path():
    codes = fp8_codes((24, 2048 + 64), seed=11)
    s = np.float32(2.0 ** -5)
    vals = torch_e4m3_values(codes) * s                 # exact: 4 significant bits, scaled by a power of two
    bits = float32_to_bf16_bits(vals)
    assert np.array_equal(bf16_to_float32(bits), vals)  # exactly representable in bf16
    a, b = oracle.quantize_fp8(codes, s), oracle.quantize(bits)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_quantize_fp8_rounds_each_product_once_to_fp32():
    codes = fp8_codes((16, 1024 + 32), seed=12)
    for s in (np.float32(0.0137), np.float32(3.3e-3), np.float32(1.7e3)):
        vals = (torch_e4m3_values(codes) * s).astype(np.float32)   # numpy: one fp32 rounding per product
        a, b = oracle.quantize_fp8(codes, s), oracle.quantize_f32(vals)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_quantize_fp8_sign_and_zero_scale():
    codes = fp8_codes((8, 512), seed=13)
    s = np.float32(0.021)
    pos, neg = oracle.quantize_fp8(codes, s), oracle.quantize_fp8(codes, -s)
    # every value changes sign (zeros too: 0 * -s = -0), so every code's sign bit flips
    assert np.array_equal(neg[0], pos[0] ^ 0x88) and np.array_equal(neg[1], pos[1]) and neg[2] == pos[2]
    z = oracle.quantize_fp8(codes, np.float32(0.0))
    assert not z[0].any() and not z[1].any() and z[2] == 0.0


def test_quantize_f32_entry_equals_bf16_entry():
    bits = tensor_bits(workload("gemv_1024").tensor("w"))[:64]
    a, b = oracle.quantize_f32(bf16_to_float32(bits)), oracle.quantize(bits)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


# ------------------------------------------- fused neighbours: SwiGLU, RMSNorm
def test_silu_closed_forms_and_identities():
    """silu(z) = z * sigmoid(z). At z = ln k the sigmoid is exactly k/(k+1);
    the sigmoid's symmetry gives silu(z) - silu(-z) = z; the minimum of silu
    is -W0(1/e) (Lambert W), taken at z = -1 - W0(1/e); silu(z) -> z for
    large z and -> 0 for very negative z."""
    for k in (2.0, 3.0, 7.0, 0.5, 100.0):
        z = np.log(k)
        assert oracle.silu(z) == pytest.approx(z * k / (k + 1), rel=1e-14)
    zs = np.linspace(-30, 30, 6001)
    h = oracle.swiglu(zs, np.ones_like(zs))                      # silu itself at u = 1
    assert np.allclose(h - oracle.swiglu(-zs, np.ones_like(zs)), zs, rtol=1e-14, atol=1e-14)
    from scipy.special import lambertw
    w = float(lambertw(np.exp(-1.0)).real)
    grid = np.linspace(-3.0, 1.0, 400001)
    v = oracle.swiglu(grid, np.ones_like(grid))
    assert v.min() == pytest.approx(-w, abs=1e-10)
    assert grid[v.argmin()] == pytest.approx(-1.0 - w, abs=2e-5)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(60.0) == pytest.approx(60.0, rel=1e-15)
    assert 0.0 >= oracle.silu(-60.0) > -1e-23


def test_swiglu_gates_the_up_product_with_silu_of_the_gate():
    """h(g, u) is silu(g) at u = 1 (pinned above), linear in u, zero for a
    zero gate whatever u is, and not symmetric in its operands."""
    rng = np.random.default_rng(21)
    g, u = rng.normal(0, 3, 1000), rng.normal(0, 3, 1000)
    h = oracle.swiglu(g, u)
    assert np.allclose(oracle.swiglu(g, 2 * u), 2 * h, rtol=1e-15)
    assert np.allclose(h, oracle.swiglu(g, np.ones_like(g)) * u, rtol=1e-15)
    assert np.all(oracle.swiglu(np.zeros_like(u), u) == 0)
    assert not np.allclose(h, oracle.swiglu(u, g))


def test_rmsnorm_properties_and_a_closed_form():
    """Rows come out with unit mean square (gain 1, eps 0), point the same way
    as the input, do not change when the row is scaled by a power of two or
    repeated (a mean, not a sum), and the gain multiplies each column. With
    eps = 1e-6 a row of +-1 maps to +-1/sqrt(1 + 1e-6); a zero row stays zero."""
    x = bf16_tensor((6, 96), 31, 1.5)
    ones = float32_to_bf16_bits(np.ones(96, np.float32))
    out = oracle.rmsnorm(x, ones, 0.0)
    assert np.allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-14)
    xf = bf16_to_float32(x).astype(np.float64)
    nz = xf != 0
    ratio = np.where(nz, out / np.where(nz, xf, 1.0), np.nan)
    for m in range(6):
        r = ratio[m][nz[m]]
        assert np.all(r > 0) and np.allclose(r, r[0], rtol=1e-15)
    assert np.array_equal(oracle.rmsnorm(float32_to_bf16_bits((xf * 4).astype(np.float32)), ones, 0.0), out)
    twice = np.concatenate([x, x], axis=1)
    ones2 = float32_to_bf16_bits(np.ones(192, np.float32))
    assert np.allclose(oracle.rmsnorm(twice, ones2, 0.0)[:, :96], out, rtol=1e-15)
    gain = bf16_tensor((96,), 32, 1.0)
    assert np.allclose(oracle.rmsnorm(x, gain, 0.0), out * bf16_to_float32(gain)[None, :], rtol=1e-15)
    pm = float32_to_bf16_bits(np.array([[1, -1, 1, -1, -1, 1, 1, 1]], np.float32))
    ones8 = float32_to_bf16_bits(np.ones(8, np.float32))
    expect = 0.99999950000037499969        # 1 / sqrt(1.000001)
    assert np.allclose(oracle.rmsnorm(pm, ones8, 1e-6)[0], expect * bf16_to_float32(pm)[0].astype(np.float64),
                       rtol=1e-15, atol=0)
    z = np.zeros((2, 32), np.uint16)
    assert np.all(oracle.rmsnorm(z, float32_to_bf16_bits(np.ones(32, np.float32)), 1e-6) == 0)


def test_gemv_f64_equals_bf16_entry_and_numpy():
    """The fp64-activation product equals the bf16 one on bf16-valued rows
    (same sums in the same order) and numpy's float64 matmul of the
    dequantised weights on arbitrary fp64 rows."""
    rng = np.random.default_rng(33)
    W = float32_to_bf16_bits(rng.normal(0, 0.05, (40, 1056)).astype(np.float32))
    p, s, g = oracle.quantize(W)
    xb = float32_to_bf16_bits(rng.normal(0, 1, (3, 1056)).astype(np.float32))
    y1, l1 = oracle.gemv(xb, p, s, g)
    y2, l2 = oracle.gemv_f64(bf16_to_float32(xb).astype(np.float64), p, s, g)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)
    xd = rng.normal(0, 1, (4, 1056))
    D = dequant_from_bits(p, s, g)
    y3, l3 = oracle.gemv_f64(xd, p, s, g)
    assert np.allclose(y3, xd @ D.T, rtol=1e-12, atol=1e-14 * np.abs(D).sum())
    assert np.allclose(l3, np.abs(xd) @ np.abs(D).T, rtol=1e-12)


# ------------------------------------------------------------------- MXFP4
def load_mx_example():
    rows, codes, scales = [], [], []
    with open(os.path.join(GOLDEN, "mx_worked_example.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "row":
                rows.append([float(v) for v in vals])
            elif key == "codes":
                codes.append([int(v, 16) for v in vals])
            elif key == "scales":
                scales.append([int(v, 16) for v in vals])
    W = np.array(rows, dtype=np.float32)
    Wb = float32_to_bf16_bits(W)
    assert np.array_equal(bf16_to_float32(Wb), W) and np.array_equal(np.signbit(bf16_to_float32(Wb)), np.signbit(W))
    c = np.array(codes, np.uint8)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)   # even k in the low nibble
    return Wb, packed, np.array(scales, np.uint8)


def test_e8m0_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for c in range(256):
        v = oracle.e8m0_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c] == 2.0 ** (c - 127), c


def test_mx_quantize_worked_example():
    Wb, packed, scales = load_mx_example()
    p, s = oracle.mx_quantize(Wb)
    assert np.array_equal(s, scales), (s, scales)
    assert np.array_equal(p, packed), np.flatnonzero(p != packed)


def test_mx_round_trip_and_bounds():
    """Blocks built from E2M1 values times a power of two whose largest
    magnitude is 4 or 6 times it quantise back to themselves exactly; on
    random bf16 weights every unclamped block has 4 X <= amax < 8 X
    (X = E8M0 of its scale), its largest element encodes to 4 or 6, and
    every element is within 2 X of its dequantised value."""
    rng = np.random.default_rng(41)
    N, K = 16, 256
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    codes = rng.integers(0, 8, (N, K))
    codes[:, ::32] = rng.choice([6, 7], (N, K // 32))        # each block's amax is 4 or 6 units
    shared = rng.integers(-20, 20, (N, K // 32))
    sign = rng.choice([-1.0, 1.0], (N, K))
    W = sign * mags[codes] * np.repeat(2.0 ** shared, 32, axis=1)
    Wb = float32_to_bf16_bits(W.astype(np.float32))
    p, s = oracle.mx_quantize(Wb)
    assert np.array_equal(s, (shared + 127).astype(np.uint8))
    assert np.array_equal(oracle.mx_dequant(p, s), bf16_to_float32(Wb).astype(np.float64))
    Wr = bf16_tensor((64, 512), 42, 0.02, outlier_p=0.01, outlier_scale=20.0)
    p, s = oracle.mx_quantize(Wr)
    X = np.array([[oracle.e8m0_value(c) for c in row] for row in s])
    w = bf16_to_float32(Wr).astype(np.float64).reshape(64, 16, 32)
    amax = np.abs(w).max(axis=2)
    assert np.all((4 * X <= amax) & (amax < 8 * X))
    D = oracle.mx_dequant(p, s).reshape(64, 16, 32)
    assert np.all(np.abs(w - D) <= 2 * X[:, :, None])
    at = np.abs(w).argmax(axis=2)
    amax_code = np.take_along_axis((p[:, :, None] >> np.array([0, 4])).reshape(64, 16, 32) & 7, at[:, :, None], 2)
    assert np.all(np.isin(amax_code, [6, 7]))


def mx_dequant_from_bits(p, s):
    e2 = np.array([float(minifloat_value(c, 2, 1, 1)) for c in range(16)])
    e8 = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e8m0fnu).double().numpy()
    q = np.stack([p & 15, p >> 4], axis=2).reshape(p.shape[0], -1)
    return e2[q] * np.repeat(e8, 32, axis=1)


def test_mx_gemv_matches_numpy_on_tiny_matrices():
    rng = np.random.default_rng(43)
    for N, K, M in [(1, 32, 1), (3, 64, 2), (9, 1024 + 32, 3)]:
        W = float32_to_bf16_bits(rng.normal(0, 0.05, (N, K)).astype(np.float32))
        x = float32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
        p, s = oracle.mx_quantize(W)
        D = mx_dequant_from_bits(p, s)
        assert np.array_equal(oracle.mx_dequant(p, s), D)
        xf = bf16_to_float32(x).astype(np.float64)
        y, l1 = oracle.mx_gemv(x, p, s)
        assert np.allclose(y, xf @ D.T, rtol=1e-13, atol=1e-15 * np.abs(D).sum())
        assert np.allclose(l1, np.abs(xf) @ np.abs(D).T, rtol=1e-13)


def test_mx_a4_product_matches_bit_field_decodes():
    """Both operands MXFP4: the product equals the one built from decodes
    that do not use the oracle (E2M1 bit fields, E8M0 through
    torch.float8_e8m0fnu), and not the one with an operand's K order
    reversed."""
    rng = np.random.default_rng(45)
    for M, N, K in [(1, 1, 32), (2, 3, 64), (5, 9, 1024 + 32)]:
        x = float32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
        W = float32_to_bf16_bits(rng.normal(0, 0.05, (N, K)).astype(np.float32))
        xp, xs = oracle.mx_quantize(x)
        wp, ws = oracle.mx_quantize(W)
        A, B = mx_dequant_from_bits(xp, xs), mx_dequant_from_bits(wp, ws)
        y, l1 = oracle.mx_a4_product(xp, xs, wp, ws)
        assert np.allclose(y, A @ B.T, rtol=1e-13, atol=1e-15 * (np.abs(A) @ np.abs(B).T).max())
        assert np.allclose(l1, np.abs(A) @ np.abs(B).T, rtol=1e-13)
        if K > 32:
            assert not np.allclose(y, A[:, ::-1] @ B.T)


def test_mx_a4_product_equals_the_bf16_product_on_representable_activations():
    """Activations that MXFP4 holds exactly (per 32-block: E2M1 values times
    2^e with a block maximum of 4 or 6, so the shared exponent is e) round-trip
    through mx_quantize, and then the product of the two MXFP4 operands equals
    the oracle's MXFP4 x bf16 product (its C path) up to the order of fp64
    sums."""
    rng = np.random.default_rng(46)
    vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    M, N, K = 3, 7, 96
    x = rng.choice(vals, (M, K)) * rng.choice([-1, 1], (M, K))
    x = x.reshape(M, K // 32, 32)
    x[:, :, 0] = rng.choice([4.0, -6.0, 6.0, -4.0], (M, K // 32))   # the block maximum
    x = (x * 2.0 ** rng.integers(-6, 7, (M, K // 32, 1))).reshape(M, K)
    xb = float32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_to_float32(xb).astype(np.float64), x)
    xp, xs = oracle.mx_quantize(xb)
    assert np.array_equal(oracle.mx_dequant(xp, xs), x)
    W = float32_to_bf16_bits(rng.normal(0, 0.05, (N, K)).astype(np.float32))
    wp, ws = oracle.mx_quantize(W)
    y, l1 = oracle.mx_a4_product(xp, xs, wp, ws)
    y2, l2 = oracle.mx_gemv(xb, wp, ws)
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-15 * l2.max())
    assert np.allclose(l1, l2, rtol=1e-13)


def test_mx_a4_product_exact_against_rationals():
    """One row of x and one weight row of 32 elements each, the weight from
    the MXFP4 worked example: every product and sum is a short binary
    fraction, so the fp64 result equals exact rational arithmetic over the
    codes' bit-field values and the scales' exponents."""
    Wb, wp, ws = load_mx_example()
    rng = np.random.default_rng(47)
    K = wp.shape[1] * 2
    xv = rng.choice([0, .5, 1, 1.5, 2, 3, 4, 6], (1, K)) * rng.choice([-1, 1], (1, K))
    xv.reshape(1, K // 32, 32)[:, :, 0] = 6.0
    xb = float32_to_bf16_bits((xv * 2.0 ** -3).astype(np.float32))
    xp, xs = oracle.mx_quantize(xb)
    y, _ = oracle.mx_a4_product(xp, xs, wp, ws)
    e2 = [minifloat_value(c, 2, 1, 1) for c in range(16)]
    for n in range(wp.shape[0]):
        acc = Fraction(0)
        for k in range(K):
            qa = xp[0, k // 2] >> (4 * (k % 2)) & 15
            qw = wp[n, k // 2] >> (4 * (k % 2)) & 15
            acc += (e2[qa] * Fraction(2) ** (int(xs[0, k // 32]) - 127)) * (e2[qw] * Fraction(2) ** (int(ws[n, k // 32]) - 127))
        assert y[0, n] == float(acc)


def test_mx_tile_matches_reshape_formulation():
    """The MXFP4 device layout written as array reshapes: codes as in the
    NVFP4 tile; scale (row 8g + 2i + h, block 32c + l) at 4096 + 128h + 4l + i."""
    rng = np.random.default_rng(44)
    for N, K in [(8, 1024), (13, 2080), (1, 32)]:
        p = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = rng.integers(0, 255, (N, K // 32), dtype=np.uint8)
        G, C = (N + 7) // 8, (K + 1023) // 1024
        pp = np.zeros((G * 8, C * 512), np.uint8)
        pp[:N, :K // 2] = p
        ss = np.zeros((G * 8, C * 32), np.uint8)
        ss[:N, :K // 32] = s
        codes = pp.reshape(G, 8, C, 512).transpose(0, 2, 1, 3).reshape(G, C, 4096)
        sc = ss.reshape(G, 4, 2, C, 32).transpose(0, 3, 2, 4, 1).reshape(G, C, 256)   # [g][c][h][l][i]
        ref = np.concatenate([codes, sc], axis=2).reshape(-1)
        assert np.array_equal(oracle.mx_tile(p, s), ref), (N, K)
