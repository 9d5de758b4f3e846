"""Pins for the oracle's output RMS normalisation and its backward."""
import numpy as np

import oracle


def test_constant_row_closed_form():
    # x = c 1: mean(x^2) = c^2, so y = c / sqrt(c^2 + eps) * weight
    g = np.array([1.0, -2.0, 0.5, 3.0])
    for c, eps in ((2.0, 1e-6), (-0.3, 0.01), (1e-4, 1e-6)):
        y = oracle.rmsnorm(np.full((1, 4), c), g, eps=eps)
        np.testing.assert_allclose(y[0], c / np.sqrt(c * c + eps) * g, rtol=1e-14)


def test_unit_rms_and_scale_invariance_without_eps():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 5, 2, 16)) * rng.uniform(0.1, 10.0, (3, 5, 2, 1))
    y = oracle.rmsnorm(x, None, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, None, eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(oracle.rmsnorm(-x, None, eps=0.0), -y, rtol=1e-14)
    g = rng.standard_normal(16)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, eps=0.0), y * g, rtol=1e-14)
    # a zero row stays zero with eps > 0
    assert np.all(oracle.rmsnorm(np.zeros((1, 8)), np.ones(8), eps=1e-6) == 0.0)


def test_one_element_row_is_the_sign():
    # d = 1: y = x / sqrt(x^2) = sign(x) at eps = 0
    x = np.array([[3.0], [-0.25]])
    np.testing.assert_array_equal(oracle.rmsnorm(x, None, eps=0.0), [[1.0], [-1.0]])


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((2, 3, 8)) * 2.0
    g = rng.standard_normal(8)
    dy = rng.standard_normal((2, 3, 8))
    eps = 1e-3
    got = oracle.rmsnorm_backward(x, g, dy, eps=eps)
    loss = lambda xx, gg: float(np.sum(dy * oracle.rmsnorm(xx, gg, eps=eps)))
    h = 1e-6
    fx = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        e = np.zeros_like(x)
        e[i] = h
        fx[i] = (loss(x + e, g) - loss(x - e, g)) / (2 * h)
    fg = np.zeros_like(g)
    for j in range(8):
        e = np.zeros_like(g)
        e[j] = h
        fg[j] = (loss(x, g + e) - loss(x, g - e)) / (2 * h)
    np.testing.assert_allclose(got["dx"], fx, rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(got["dweight"], fg, rtol=1e-7, atol=1e-8)


def test_backward_is_orthogonal_to_the_row_without_eps():
    # y does not change along x when eps = 0 (scale invariance), so dx . x = 0 per row
    rng = np.random.default_rng(43)
    x = rng.standard_normal((4, 32))
    dx = oracle.rmsnorm_backward(x, rng.standard_normal(32), rng.standard_normal((4, 32)), eps=0.0)["dx"]
    np.testing.assert_allclose(np.sum(dx * x, axis=-1), 0.0, atol=1e-13)
