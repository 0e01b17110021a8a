"""Pins of the oracle's fp16 conversion and Hadamard matrix against library
routines (numpy's IEEE half conversion, scipy's Sylvester Hadamard)."""
import numpy as np
import pytest
import scipy.linalg

import oracle


def test_h2d_matches_numpy_on_every_finite_half():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_d2h_round_to_nearest_even_matches_numpy():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        # exact midpoints between neighbouring halves: ties must go to even
        (np.arange(0, 0x7bff, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
         + np.arange(1, 0x7c00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2,
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -25, 2.0 ** -24 * 1.5, 5.96e-8]),
    ])
    vals = np.concatenate([vals, -vals])
    ref = vals.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_f16(vals)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_matrix_is_scipy_sylvester(d):
    H = oracle.hadamard_matrix(d)
    assert np.array_equal(H * np.sqrt(d), scipy.linalg.hadamard(d).astype(np.float64))


def test_hadamard_orthonormal_involution_and_e0():
    d = 128
    H = oracle.hadamard_matrix(d)
    assert np.allclose(H @ H, np.eye(d), atol=1e-13)
    e0 = np.zeros(d); e0[0] = 1.0
    assert np.allclose(oracle.hadamard(e0), np.full(d, 1 / np.sqrt(d)), atol=1e-15)
    w = np.random.default_rng(1).standard_normal(d)
    u = oracle.hadamard(w)
    assert abs(np.linalg.norm(u) - np.linalg.norm(w)) < 1e-12 * np.linalg.norm(w)
    assert np.allclose(oracle.hadamard(u), w, atol=1e-12)
    # integer vector: unnormalised transform twice gives d * identity exactly
    wi = np.random.default_rng(2).integers(-8, 8, d).astype(np.float64)
    Hi = scipy.linalg.hadamard(d).astype(np.float64)
    assert np.array_equal(Hi @ (Hi @ wi), d * wi)
    assert np.allclose(oracle.hadamard(wi) * np.sqrt(d), Hi @ wi, atol=1e-12)
