"""Pins of the oracle's k-means: Lloyd's monotonicity and fixed point, closed
forms in one dimension, and the Gaussian rate-distortion bounds that any
codebook at 2 and 1 bits per element must respect."""
import numpy as np
import pytest

import oracle
from kv_cache_bit_amd import synth


def test_distortion_non_increasing_and_fixed_point():
    x = synth.randn_samples(3, 4096, 4).numpy()
    cent, cb, dist = oracle.kmeans(x, 32, 60)
    assert np.all(np.diff(dist) <= 1e-15)
    # at convergence every centroid is the mean of the samples nearest to it
    d2 = ((x[:, None, :].astype(np.float64) - cent[None]) ** 2).sum(-1)
    a = np.argmin(d2, 1)
    for k in range(32):
        m = x[a == k].astype(np.float64)
        if len(m):
            assert np.allclose(cent[k], m.mean(0), atol=1e-10)
    assert np.array_equal(cb, oracle.f64_to_f16(cent))


def test_single_centroid_is_the_mean_and_explicit_init():
    x = synth.randn_samples(4, 1000, 8).numpy()
    cent, _, dist = oracle.kmeans(x, 1, 2)
    assert np.allclose(cent[0], x.astype(np.float64).mean(0), atol=1e-12)
    assert dist[0] == pytest.approx(((x.astype(np.float64) - x[0]) ** 2).sum() / x.size, rel=1e-12)
    init = np.zeros((1, 8))
    cent2, _, dist2 = oracle.kmeans(x, 1, 1, init=init)
    assert dist2[0] == pytest.approx((x.astype(np.float64) ** 2).sum() / x.size, rel=1e-12)


def test_one_bit_scalar_lloyd_max():
    """Two centroids on N(0,1) converge to +-sqrt(2/pi) with MSE 1 - 2/pi."""
    x = synth.randn_samples(5, 1 << 18, 1).numpy()
    cent, _, dist = oracle.kmeans(x, 2, 30, init=np.array([[-0.1], [0.1]]))
    assert np.allclose(np.sort(cent[:, 0]), [-np.sqrt(2 / np.pi), np.sqrt(2 / np.pi)], atol=2e-2)
    assert dist[-1] == pytest.approx(1 - 2 / np.pi, abs=1e-2)


@pytest.mark.parametrize("bits,s,lloyd_max", [(2, 4, 0.1175), (1, 8, 1 - 2 / np.pi)])
def test_gaussian_rate_distortion_bounds(bits, s, lloyd_max):
    """256 codewords over s dims is `bits` bits per element.  On held-out
    N(0,1) data the per-element MSE lies above Shannon's D(R) = 2^(-2 bits)
    and below the product of scalar Lloyd-Max quantisers (a valid 256-word
    codebook, so a converged k-means should not do worse)."""
    x = synth.randn_samples(10 + bits, 1 << 16, s).numpy()
    cent, cb, dist = oracle.kmeans(x, 256, 40)
    test = synth.randn_samples(20 + bits, 1 << 15, s).numpy().astype(np.float64)
    cbd = oracle.f16_to_f64(cb)
    d2 = ((test[:, None, :] - cbd[None]) ** 2).sum(-1).min(1)
    mse = d2.sum() / test.size
    assert mse > 2.0 ** (-2 * bits)
    assert mse < lloyd_max * 1.02
