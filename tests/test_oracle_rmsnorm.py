"""Pins for the oracle's output RMS normalisation and its backward, and planted mistakes in a
copy of them that the pins must catch."""
import inspect

import numpy as np
import pytest

import oracle


def pin_constant_row(f, fb):
    # x = c 1: mean(x^2) = c^2, so y = c / sqrt(c^2 + eps) * weight
    g = np.array([1.0, -2.0, 0.5, 3.0])
    for c, eps in ((2.0, 1e-6), (-0.3, 0.01), (1e-4, 1e-6)):
        y = f(np.full((1, 4), c), g, eps=eps)
        np.testing.assert_allclose(y[0], c / np.sqrt(c * c + eps) * g, rtol=1e-14)


def pin_unit_rms_and_scale_invariance(f, fb):
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 5, 2, 16)) * rng.uniform(0.1, 10.0, (3, 5, 2, 1))
    y = f(x, None, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(f(7.5 * x, None, eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(f(-x, None, eps=0.0), -y, rtol=1e-14)
    g = rng.standard_normal(16)
    np.testing.assert_allclose(f(x, g, eps=0.0), y * g, rtol=1e-14)
    # a zero row stays zero with eps > 0
    assert np.all(f(np.zeros((1, 8)), np.ones(8), eps=1e-6) == 0.0)


def pin_one_element_row_is_the_sign(f, fb):
    # d = 1: y = x / sqrt(x^2) = sign(x) at eps = 0
    x = np.array([[3.0], [-0.25]])
    np.testing.assert_array_equal(f(x, None, eps=0.0), [[1.0], [-1.0]])


def pin_backward_matches_finite_differences(f, fb):
    rng = np.random.default_rng(42)
    x = rng.standard_normal((2, 3, 8)) * 2.0
    g = rng.standard_normal(8)
    dy = rng.standard_normal((2, 3, 8))
    eps = 1e-3
    got = fb(x, g, dy, eps=eps)
    loss = lambda xx, gg: float(np.sum(dy * f(xx, gg, eps=eps)))
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


def pin_backward_orthogonal_to_the_row(f, fb):
    # y does not change along x when eps = 0 (scale invariance), so dx . x = 0 per row
    rng = np.random.default_rng(43)
    x = rng.standard_normal((4, 32))
    dx = fb(x, rng.standard_normal(32), rng.standard_normal((4, 32)), eps=0.0)["dx"]
    np.testing.assert_allclose(np.sum(dx * x, axis=-1), 0.0, atol=1e-13)


PINS = [pin_constant_row, pin_unit_rms_and_scale_invariance, pin_one_element_row_is_the_sign,
        pin_backward_matches_finite_differences, pin_backward_orthogonal_to_the_row]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.rmsnorm, oracle.rmsnorm_backward)


# one textual change each to a copy of rmsnorm ("f") or rmsnorm_backward ("b")
MUTANTS = {
    "mean_as_sum": ("f", "np.mean(x * x, axis=-1, keepdims=True) + eps", "np.sum(x * x, axis=-1, keepdims=True) + eps"),
    "eps_dropped": ("f", "keepdims=True) + eps)", "keepdims=True))"),
    "sqrt_dropped": ("f", "1.0 / np.sqrt(np.mean(", "1.0 / (np.mean("),
    "weight_ignored": ("f", "return y if weight is None else y * _f64(weight)", "return y"),
    "mean_term_dropped": ("b", "dx = r * (u - xh * np.mean(xh * u, axis=-1, keepdims=True))", "dx = r * u"),
    "weight_dropped_in_dx": ("b", "u = dy * g", "u = dy"),
    "dweight_of_raw_x": ("b", "dweight = (dy * xh)", "dweight = (dy * x)"),
    "scale_dropped_in_dx": ("b", "dx = r * (u", "dx = (u"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    which, old, new = MUTANTS[name]
    srcs = {"f": inspect.getsource(oracle.rmsnorm), "b": inspect.getsource(oracle.rmsnorm_backward)}
    assert srcs[which].count(old) == 1, f"mutation anchor for {name} not found exactly once"
    srcs[which] = srcs[which].replace(old, new)
    ns = {"np": np, "_f64": oracle._f64}
    exec(srcs["f"], ns)
    exec(srcs["b"], ns)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):  # a mutant may divide a zero row by zero
                pin(ns["rmsnorm"], ns["rmsnorm_backward"])
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches {name}"
