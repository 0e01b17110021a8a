"""Pins of the oracle's cosine refinement of the codebook (technical summary
sec. 3, Codebook Construction): the analytic gradient against central finite
differences, descent for a small step, an exact fixed point, and the held-out
gain that the pages report as helpful."""
import numpy as np

import oracle
from kv_cache_bit_amd import synth

D = 128


def _start(bits, s):
    cent, _, _ = oracle.kmeans(synth.randn_samples(bits, 1 << 13, s).numpy(), 256, 6)
    return cent


def test_gradient_matches_finite_differences():
    x = synth.randn_samples(11, 64, D).numpy()
    c = _start(2, 4)
    loss, g = oracle.cos_loss_grad(x, c)
    assert 0.0 < loss < 0.2
    rng = np.random.default_rng(0)
    used = np.flatnonzero(np.abs(g).sum(1) > 0)
    checked = 0
    for k in rng.choice(used, 12, replace=False):
        for e in range(4):
            h = 1e-6
            cp, cm = c.copy(), c.copy()
            cp[k, e] += h
            cm[k, e] -= h
            lp, _ = oracle.cos_loss_grad(x, cp)
            lm, _ = oracle.cos_loss_grad(x, cm)
            fd = (lp - lm) / (2 * h)
            # the assignment is piecewise constant; a step that crosses a
            # Voronoi boundary shows up as a jump far larger than the slope
            if abs(fd - g[k, e]) > 1e-3:
                continue
            assert abs(fd - g[k, e]) <= 1e-6 + 1e-4 * abs(g[k, e])
            checked += 1
    assert checked >= 40


def test_descent_and_fixed_point():
    x = synth.randn_samples(12, 256, D).numpy()
    c = _start(1, 8)
    _, _, loss = oracle.finetune(x, c, 6, 4.0)
    assert np.all(np.diff(loss) < 0)
    # vectors built from codewords are quantised exactly: loss 0, no gradient
    rng = np.random.default_rng(1)
    cb = oracle.f16_to_f64(oracle.f64_to_f16(c))
    xs = cb[rng.integers(0, 256, (32, D // 8))].reshape(32, D).astype(np.float32)
    l0, g0 = oracle.cos_loss_grad(xs, cb)
    assert abs(l0) < 1e-12 and np.abs(g0).max() < 1e-12
    c1, _, _ = oracle.finetune(xs, cb, 3, 10.0)
    assert np.array_equal(c1, cb)


def test_refinement_lowers_held_out_cosine_distance():
    for bits, s in ((2, 4), (1, 8)):
        c = _start(bits, s)
        x = synth.randn_samples(20 + bits, 1024, D).numpy()
        xt = synth.randn_samples(30 + bits, 1024, D).numpy()
        c2, _, loss = oracle.finetune(x, c, 12, 64.0)
        assert loss[-1] < loss[0]
        l0, _ = oracle.cos_loss_grad(xt, c)
        l1, _ = oracle.cos_loss_grad(xt, c2)
        assert l1 < l0
