"""Pins of the oracle's Hadamard rotation and power-of-two block scales
(page "Sparse latent attention": the indexer's q and k are multiplied by
H_128 / sqrt(128) before quantisation; page "Rotate first features":
rotate_activation ahead of act_quant with its scale_fmt option)."""
import numpy as np
import pytest
import scipy.linalg

import oracle



def _rows(seed, n, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((n, 128)) * scale).astype(np.float32)


def test_hadamard_matches_library_matrix_product():
    # scipy's Sylvester Hadamard matrix in a float64 product: the oracle's
    # output is that value rounded once to float32 (a double rounding through
    # the float64 sum could move it by at most one float32 unit)
    x = _rows(0, 64)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(128).astype(np.float64).T / np.sqrt(128.0)
    got = oracle.hadamard(x)
    assert got.dtype == np.float32
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 2.0 ** -24 * np.abs(ref))
    assert np.mean(got == ref.astype(np.float32)) > 0.999


def test_hadamard_worked_example():
    # x = (1, 2, ..., 128): H x / sqrt(128) has y[0] = 8256 / sqrt(128) (the
    # sum 1 + ... + 128) and, for i = 2^m, y[i] = -(2^m * 64) / sqrt(128)
    # (the row of H for a power of two alternates in blocks of 2^m, and each
    # block pair differs by 2^m in each of its 64 terms)
    x = np.arange(1, 129, dtype=np.float32)[None]
    y = oracle.hadamard(x).astype(np.float64)[0] * np.sqrt(128.0)
    assert abs(y[0] - 8256.0) <= 1e-3
    for m in range(7):
        assert abs(y[1 << m] + (1 << m) * 64.0) <= 1e-3, m
    # every other index (not 0, not a power of two) sums to zero
    others = [i for i in range(1, 128) if i & (i - 1)]
    assert np.all(np.abs(y[others]) <= 1e-3)


def test_hadamard_unit_vectors_and_signs():
    e = np.eye(128, dtype=np.float32)
    got = oracle.hadamard(e).astype(np.float64) * np.sqrt(128.0)
    # row i of the result is column i of H_128 = (-1)^popcount(i & j)
    j = np.arange(128)
    expect = np.array([[(-1.0) ** bin(i & jj).count("1") for jj in j] for i in range(128)])
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-6)
    # e_0 maps to the constant vector 128^-0.5
    np.testing.assert_allclose(oracle.hadamard(e[:1]), np.full((1, 128), 128 ** -0.5), rtol=1e-7)


def test_hadamard_is_orthonormal_involution():
    x = _rows(1, 32, 3.0)
    y = oracle.hadamard(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    np.testing.assert_allclose(oracle.hadamard(y), x, rtol=0, atol=1e-5 * np.abs(x).max())


def test_hadamard_bf16_output_is_rounded_float32_result():
    x = _rows(2, 16)
    np.testing.assert_array_equal(oracle.hadamard(x, out_bf16=True),
                                  oracle.round_bf16(oracle.hadamard(x)))


def test_hadamard_leaves_exact_indexer_scores_unchanged():
    # orthonormal: q.k is preserved, so ReLU(q.k) and the score are too
    q, k = _rows(3, 8).astype(np.float64), _rows(4, 8).astype(np.float64)
    H = scipy.linalg.hadamard(128) / np.sqrt(128.0)
    np.testing.assert_allclose((q @ H.T) @ (k @ H.T).T, q @ k.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("scale", [1e-6, 0.3, 1.0, 17.0, 3e4])
def test_pow2_scales(scale):
    x = _rows(5, 256, scale)
    x[0] = 0.0
    codes, s = oracle.quantize(x, pow2=True)
    amax = np.abs(x).max(axis=1)
    base = (amax / np.float32(448.0)).astype(np.float32)
    m, _ = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)                                   # powers of two
    nz = amax > 0
    assert np.all(s[nz] >= base[nz]) and np.all(s[nz] < 2 * base[nz])
    assert s[0] == 1.0
    assert np.all(np.abs(x[nz]) / s[nz, None] <= 448.0)
    # codes are the E4M3 encodings of the exact quotients
    np.testing.assert_array_equal(codes, oracle.e4m3_encode(x / s[:, None]))


def test_pow2_scale_of_exact_power_of_two_is_itself():
    x = np.zeros((1, 128), np.float32)
    x[0, 5] = 448.0 * 2.0 ** -3
    _, s = oracle.quantize(x, pow2=True)
    assert s[0] == 2.0 ** -3
