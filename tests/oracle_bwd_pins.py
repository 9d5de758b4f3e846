"""Pins for the oracle's backward (reverse mode of the recurrence).

Each pin takes `backward(q, k, v, alpha, b, w, S0, dO, dS_T) -> dict` and the oracle's forward
(pinned on its own by tests/oracle_pins.py), so the same pins run on the oracle and on broken
copies of it (tests/test_oracle_bwd.py). None re-types the oracle's adjoint loop: they compare it
with finite differences of the forward, a closed form for one token, the affine dependence of the
loss on S0, and automatic differentiation of an explicit transition-matrix recurrence.

The loss is L = sum_t <dO_t, o_t> + <dS_T, S_T>; the update rule is the one on the page
"NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph "Техническая схема".
"""
from __future__ import annotations

import numpy as np

from oracle_pins import random_inputs

NAMES = ("q", "k", "v", "alpha", "b", "w")
GRAD = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "b": "db", "w": "dw"}


def loss(forward, xs, S0, dO, dST):
    o, S_T = forward(*xs, S0)
    L = float(np.sum(dO * o))
    if dST is not None:
        L += float(np.sum(dST * S_T))
    return L


def pin_bwd_finite_differences(backward, forward, seed=11):
    """Central differences of L through the forward, every input element, at a length that
    crosses the 64-token checkpoint boundary (T = 70) and at a short one."""
    for T, dk, dv in ((5, 3, 4), (70, 2, 3)):
        rng = np.random.default_rng(seed + T)
        xs = list(random_inputs(rng, 1, T, 2, dk, dv))
        S0 = xs.pop()
        dO = rng.standard_normal((1, T, 2, dv))
        dST = rng.standard_normal((1, 2, dk, dv))
        g = backward(*xs, S0, dO, dST)
        h = 1e-6
        for idx, name in enumerate(NAMES):
            x = xs[idx]
            flat = x.reshape(-1)
            picks = range(flat.size) if flat.size <= 120 else rng.choice(flat.size, 120, replace=False)
            fd = np.zeros(flat.size)
            for e in picks:
                keep = flat[e]
                flat[e] = keep + h
                Lp = loss(forward, xs, S0, dO, dST)
                flat[e] = keep - h
                Lm = loss(forward, xs, S0, dO, dST)
                flat[e] = keep
                fd[e] = (Lp - Lm) / (2 * h)
            got = g[GRAD[name]].reshape(-1)
            sel = np.array(list(picks))
            scale = max(1.0, float(np.abs(fd[sel]).max()))
            np.testing.assert_allclose(got[sel], fd[sel], rtol=0, atol=2e-7 * scale,
                                       err_msg=f"d{name} vs finite differences (T={T})")
        # dS0 likewise
        flat = S0.reshape(-1)
        fd = np.zeros(flat.size)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + h
            Lp = loss(forward, xs, S0, dO, dST)
            flat[e] = keep - h
            Lm = loss(forward, xs, S0, dO, dST)
            flat[e] = keep
            fd[e] = (Lp - Lm) / (2 * h)
        np.testing.assert_allclose(g["dS0"].reshape(-1), fd, rtol=0, atol=2e-7 * max(1.0, np.abs(fd).max()),
                                   err_msg=f"dS0 vs finite differences (T={T})")


def pin_bwd_single_token(backward, forward, seed=12):
    """One token from S0 = 0: o = u (k . q) with u = w*v, so dq = k (u . dO), dk = q (u . dO),
    dv = w*dO (k . q), dw = v*dO (k . q), db = dalpha = 0; and dS0 = Diag(alpha)
    (q - (b*k)(k . q)) dO^T (the readout cotangent pulled back through erase and decay)."""
    rng = np.random.default_rng(seed)
    q, k, v, alpha, b, w, _ = random_inputs(rng, 1, 1, 1, 4, 3, s0=False)
    dO = rng.standard_normal((1, 1, 1, 3))
    g = backward(q, k, v, alpha, b, w, None, dO, None)
    qq, kk, vv, aa, bb, ww, do = (x[0, 0, 0] for x in (q, k, v, alpha, b, w, dO))
    u = ww * vv
    kq = kk @ qq
    np.testing.assert_allclose(g["dq"][0, 0, 0], kk * (u @ do), atol=1e-14)
    np.testing.assert_allclose(g["dk"][0, 0, 0], qq * (u @ do), atol=1e-14)
    np.testing.assert_allclose(g["dv"][0, 0, 0], ww * do * kq, atol=1e-14)
    np.testing.assert_allclose(g["dw"][0, 0, 0], vv * do * kq, atol=1e-14)
    np.testing.assert_allclose(g["db"][0, 0, 0], 0.0, atol=1e-15)
    np.testing.assert_allclose(g["dalpha"][0, 0, 0], 0.0, atol=1e-15)
    dS0 = aa[:, None] * np.outer(qq - bb * kk * kq, do)
    np.testing.assert_allclose(g["dS0"][0, 0], dS0, atol=1e-14)


def pin_bwd_affine_in_initial_state(backward, forward, seed=13):
    """o and S_T are affine in S0, so L(S0) - L(0) = <dS0, S0> exactly and dS0 does not
    depend on S0."""
    rng = np.random.default_rng(seed)
    xs = list(random_inputs(rng, 2, 9, 2, 3, 4))
    S0 = xs.pop()
    dO = rng.standard_normal((2, 9, 2, 4))
    dST = rng.standard_normal((2, 2, 3, 4))
    g1 = backward(*xs, S0, dO, dST)
    g0 = backward(*xs, np.zeros_like(S0), dO, dST)
    np.testing.assert_allclose(g1["dS0"], g0["dS0"], rtol=0, atol=1e-12)
    diff = loss(forward, xs, S0, dO, dST) - loss(forward, xs, np.zeros_like(S0), dO, dST)
    np.testing.assert_allclose(float(np.sum(g1["dS0"] * S0)), diff, rtol=1e-12, atol=1e-12)


def pin_bwd_autograd(backward, forward, seed=14):
    """Automatic differentiation (torch, float64) of S_t = M_t S_{t-1} + k_t u_t^T with the
    transition matrix M_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) built explicitly."""
    import torch
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 6, 2, 3, 4
    xs = list(random_inputs(rng, B, T, H, dk, dv))
    S0 = xs.pop()
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    g = backward(*xs, S0, dO, dST)
    tx = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in xs]
    tS0 = torch.tensor(S0, dtype=torch.float64, requires_grad=True)
    q, k, v, alpha, b, w = tx
    L = torch.zeros((), dtype=torch.float64)
    eye = torch.eye(dk, dtype=torch.float64)
    for bb in range(B):
        for hh in range(H):
            S = tS0[bb, hh]
            for t in range(T):
                kt = k[bb, t, hh]
                M = (eye - torch.outer(kt, b[bb, t, hh] * kt)) @ torch.diag(alpha[bb, t, hh])
                S = M @ S + torch.outer(kt, w[bb, t, hh] * v[bb, t, hh])
                L = L + torch.dot(torch.tensor(dO[bb, t, hh]), S.T @ q[bb, t, hh])
            L = L + torch.sum(torch.tensor(dST[bb, hh]) * S)
    L.backward()
    for name, t in zip(NAMES, tx):
        np.testing.assert_allclose(g[GRAD[name]], t.grad.numpy(), rtol=0, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(g["dS0"], tS0.grad.numpy(), rtol=0, atol=1e-12, err_msg="dS0")


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_single_token, pin_bwd_affine_in_initial_state,
                pin_bwd_autograd]
