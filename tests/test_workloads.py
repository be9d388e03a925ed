"""The shared seeded input generator: C and numpy versions agree, the
rounding is round-to-nearest-even, and the distributions are as stated."""
import numpy as np

from workloads import (bf16_tensor, bf16_tensor_numpy, bf16_to_float32, float32_to_bf16_bits,
                       splitmix64, tensor_bits, workload, x_bits, WORKLOADS)
from workloads.gen import splitmix64_native


def test_splitmix64_c_matches_numpy():
    for seed in (0, 1, 0xDEADBEEFCAFEF00D):
        a = splitmix64_native(seed, 1000, 4096)
        b = splitmix64(seed, np.arange(1000, 1000 + 4096, dtype=np.uint64))
        assert np.array_equal(a, b)


def test_splitmix64_known_first_output():
    # seed 0: the first output mixes gamma itself; worked by hand from the
    # published finaliser (z ^= z>>30; z *= c1; z ^= z>>27; z *= c2; z ^= z>>31).
    z = 0x9E3779B97F4A7C15
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & (2**64 - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & (2**64 - 1)
    z ^= z >> 31
    assert int(splitmix64(0, np.array([0], np.uint64))[0]) == z == 0xE220A8397B1DCDAF


def test_bf16_tensor_c_matches_numpy_and_is_thread_independent():
    a = bf16_tensor((50, 333), 9, 0.03, start=77, outlier_p=0.01, outlier_scale=20.0, threads=1)
    b = bf16_tensor((50, 333), 9, 0.03, start=77, outlier_p=0.01, outlier_scale=20.0, threads=7)
    c = bf16_tensor_numpy((50, 333), 9, 0.03, start=77, outlier_p=0.01, outlier_scale=20.0)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -1 - 2**-8, 3.0e38], np.float32)
    assert list(float32_to_bf16_bits(f)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x7F62]
    assert np.array_equal(bf16_to_float32(np.array([0x3F80, 0xC000], np.uint16)), np.float32([1.0, -2.0]))


def test_slices_are_consistent():
    full = bf16_tensor((4, 1000), 5, 1.0)
    part = bf16_tensor((1000,), 5, 1.0, start=2000)
    assert np.array_equal(full[2], part)


def test_distributions():
    w = bf16_to_float32(tensor_bits(workload("gemv_1024").tensor("w"))).astype(np.float64)
    assert abs(w.std() - 0.02) < 2e-4 and abs(w.mean()) < 1e-4
    big = workload("dense27b_layer").tensor("down")
    d = bf16_to_float32(bf16_tensor((256, big.K), big.seed, big.sigma, 0, big.outlier_p, big.outlier_scale))
    frac = np.mean(np.abs(d) > 6 * 0.015)         # |z| > 6 sigma is ~2e-9 for a plain normal
    assert 0.0005 < frac < 0.0012
    x = bf16_to_float32(x_bits(workload("lm_head").x("x_m8"))).astype(np.float64)
    assert x.shape == (8, 1024) and abs(x.std() - 1) < 0.05
    assert not np.array_equal(x[0], x[1])


def test_workload_table_shapes():
    assert len([t for t in WORKLOADS["qwen3_0p6b_decode"].tensors]) == 28 * 7
    d = WORKLOADS["dense27b_layer"]
    assert (d.tensor("gate").N, d.tensor("gate").K, d.tensor("down").N, d.tensor("down").K) == (17408, 5120, 5120, 17408)
    assert WORKLOADS["lm_head"].tensor("w").N == 151936
    assert WORKLOADS["prefill"].x("x").M == 2048
