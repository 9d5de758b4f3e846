"""Pins for the oracle's prologue (L2 norm of q and k, sigmoid of the gate pre-activations)."""
import numpy as np
import scipy.special

import oracle


def _raw(rng, shape):
    return rng.standard_normal(shape) * rng.uniform(0.5, 4.0, shape[:-1] + (1,))


def test_l2norm_gives_unit_vectors_along_the_input():
    rng = np.random.default_rng(31)
    q, k = _raw(rng, (2, 5, 3, 8)), _raw(rng, (2, 5, 3, 8))
    a = b = np.zeros((2, 5, 3, 8))
    qn, kn, *_ = oracle.prologue(q, k, a, b, None, l2norm=True, gate_logits=False)
    for x, xn in ((q, qn), (k, kn)):
        np.testing.assert_allclose(np.linalg.norm(xn, axis=-1), 1.0, atol=1e-15)
        # parallel to the input: x = ||x|| xn
        np.testing.assert_allclose(x, np.linalg.norm(x, axis=-1, keepdims=True) * xn, atol=1e-13)
    z = np.zeros((1, 1, 1, 4))
    zn, *_ = oracle.prologue(z, z, z, z, None, l2norm=True, gate_logits=False)
    assert np.all(zn == 0.0)  # a zero vector stays zero (the 1e-12 floor)


def test_gate_logits_are_the_logistic_function():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((1, 4, 2, 6)) * 6
    q = k = np.ones_like(x)
    _, _, a, b, w = oracle.prologue(q, k, x, -x, x[..., :5], l2norm=False, gate_logits=True)
    np.testing.assert_allclose(a, scipy.special.expit(x), rtol=1e-15)
    np.testing.assert_allclose(a + b, 1.0, atol=1e-15)       # sigma(x) + sigma(-x) = 1
    np.testing.assert_allclose(w, scipy.special.expit(x[..., :5]), rtol=1e-15)
    _, _, half, _, _ = oracle.prologue(q, k, np.zeros_like(x), x, None, l2norm=False, gate_logits=True)
    assert np.all(half == 0.5)
    _, _, t, _, _ = oracle.prologue(q, k, np.full_like(x, np.log(3.0)), x, None, l2norm=False, gate_logits=True)
    np.testing.assert_allclose(t, 0.75, rtol=1e-15)


def test_prologue_off_is_the_identity():
    rng = np.random.default_rng(33)
    xs = [rng.standard_normal((1, 3, 2, 4)) for _ in range(5)]
    out = oracle.prologue(*xs, l2norm=False, gate_logits=False)
    for x, y in zip(xs, out):
        np.testing.assert_array_equal(x, y)


def test_prologue_backward_matches_finite_differences():
    # L = sum(G_out * prologue(x)) for fixed random G_out: its gradient from prologue_backward
    # against central differences of prologue() itself, for every raw input
    rng = np.random.default_rng(33)
    shp, shpv = (1, 3, 2, 5), (1, 3, 2, 4)
    raw = dict(q=_raw(rng, shp), k=_raw(rng, shp), alpha=rng.standard_normal(shp) + 2.0,
               b=rng.standard_normal(shp), w=rng.standard_normal(shpv))
    gout = dict(dq=rng.standard_normal(shp), dk=rng.standard_normal(shp), dalpha=rng.standard_normal(shp),
                db=rng.standard_normal(shp), dw=rng.standard_normal(shpv))
    names = ("q", "k", "alpha", "b", "w")

    def loss(x):
        outs = oracle.prologue(x["q"], x["k"], x["alpha"], x["b"], x["w"], l2norm=True, gate_logits=True)
        return sum(float(np.sum(gout["d" + n] * o)) for n, o in zip(names, outs))

    got = oracle.prologue_backward(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"], gout,
                                   l2norm=True, gate_logits=True)
    h = 1e-6
    for n in names:
        fd = np.zeros_like(raw[n])
        for idx in np.ndindex(raw[n].shape):
            xp = {m: v.copy() for m, v in raw.items()}
            xm = {m: v.copy() for m, v in raw.items()}
            xp[n][idx] += h
            xm[n][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        np.testing.assert_allclose(got["d" + n], fd, rtol=1e-6, atol=1e-8)


def test_prologue_backward_off_is_the_identity():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((1, 2, 1, 4))
    g = {n: rng.standard_normal((1, 2, 1, 4)) for n in ("dq", "dk", "dalpha", "db", "dw")}
    out = oracle.prologue_backward(x, x, x, x, x, g, l2norm=False, gate_logits=False)
    for n in g:
        assert np.array_equal(out[n], g[n])
