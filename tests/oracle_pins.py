"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each pin takes a `forward(q, k, v, alpha, b, w, S0) -> (o, S_T)` callable over float64
[B, T, H, d] arrays, so the same pins run on the oracle and on deliberately broken copies of
it (tests/test_oracle_mutants.py). None of them re-types the oracle's loop: each compares it
with a different formulation (hand-worked numbers, explicit transition-matrix products, closed
forms, or the scalar-gate recurrences of the earlier models).

Update rule: page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph
"Техническая схема", S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_inputs(rng, B, T, H, dk, dv, *, s0=True):
    q = _unit(rng, (B, T, H, dk))
    k = _unit(rng, (B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dv))))
    alpha = 1 / (1 + np.exp(-(rng.standard_normal((B, T, H, dk)) + 1.0)))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5 if s0 else None
    return q, k, v, alpha, b, w, S0


def pin_hand_examples(forward):
    """Hand-worked examples (tests/golden/hand_examples.json), exact up to fp64 rounding."""
    doc = json.load(open(GOLDEN, encoding="utf-8"))
    for ex in doc["examples"]:
        toks = ex["tokens"]
        arr = {n: np.array([[tk[n]] for tk in toks], dtype=np.float64)[None] for n in toks[0]}
        # arr[n]: [1, T, 1, d]
        S0 = np.array(ex["S0"], dtype=np.float64)[None, None]
        o, S_T = forward(arr["q"], arr["k"], arr["v"], arr["alpha"], arr["b"], arr["w"], S0)
        np.testing.assert_allclose(o[0, :, 0], np.array(ex["o"]), rtol=0, atol=1e-14,
                                   err_msg=ex["name"] + ": o")
        np.testing.assert_allclose(S_T[0, 0], np.array(ex["S_T"]), rtol=0, atol=1e-14,
                                   err_msg=ex["name"] + ": S_T")


def brute_force(q, k, v, alpha, b, w, S0):
    """Explicit transition matrices M_t = (I - k_t e_t^T) Diag(alpha_t), e_t = b_t*k_t.

    S_t = M_t ... M_1 S0 + sum_{j<=t} M_t ... M_{j+1} k_j u_j^T with u_j = w_j*v_j, built as
    full d_k x d_k products for every t (cubic in T; tiny inputs only).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for bb in range(B):
        for h in range(H):
            S0_bh = np.zeros((dk, dv)) if S0 is None else S0[bb, h]
            Ms = [(I - np.outer(k[bb, t, h], b[bb, t, h] * k[bb, t, h])) @ np.diag(alpha[bb, t, h])
                  for t in range(T)]
            for t in range(T):
                prod = I.copy()
                for s in range(t + 1):
                    prod = Ms[s] @ prod
                St = prod @ S0_bh
                for j in range(t + 1):
                    Pj = I.copy()
                    for s in range(j + 1, t + 1):
                        Pj = Ms[s] @ Pj
                    St = St + Pj @ np.outer(k[bb, j, h], w[bb, j, h] * v[bb, j, h])
                o[bb, t, h] = St.T @ q[bb, t, h]
                if t == T - 1:
                    S_T[bb, h] = St
    return o, S_T


def pin_brute_force(forward, seed=1):
    rng = np.random.default_rng(seed)
    for (B, T, H, dk, dv) in ((1, 6, 2, 3, 4), (2, 5, 1, 4, 2)):
        ins = random_inputs(rng, B, T, H, dk, dv)
        o, S_T = forward(*ins)
        o_ref, S_ref = brute_force(*ins)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(S_T, S_ref, rtol=0, atol=1e-12)


def pin_exact_write(forward, seed=2):
    """b = 1 and unit k: S_t^T k_t = w_t*v_t for any decay and any prior state.

    The erase removes exactly what the state returns for k_t and the write puts back the gated
    value (precise editing of the compressed memory: page "NVIDIA улучшила память LLM без роста
    затрат на контекст", section "Контекст"). Reading with q_t = k_t shows it in o_t.
    """
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 9, 2, 5, 3
    q, k, v, alpha, b, w, S0 = random_inputs(rng, B, T, H, dk, dv)
    b = np.ones_like(b)
    o, _ = forward(k, k, v, alpha, b, w, S0)
    np.testing.assert_allclose(o, w * v, rtol=0, atol=1e-13)


def pin_pure_decay(forward, seed=3):
    """b = w = 0: S_T = Diag(prod_t alpha_t) S0 and o_t = S0^T (gamma_t * q_t)."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 7, 3, 4, 6
    q, k, v, alpha, b, w, S0 = random_inputs(rng, B, T, H, dk, dv)
    b = np.zeros_like(b)
    w = np.zeros_like(w)
    o, S_T = forward(q, k, v, alpha, b, w, S0)
    gamma = np.cumprod(alpha, axis=1)  # [B, T, H, dk]
    S_ref = gamma[:, -1][..., None] * S0
    o_ref = np.einsum("bthk,bhkv->bthv", gamma * q, S0)
    np.testing.assert_allclose(S_T, S_ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)


def pin_linear_attention(forward, seed=4):
    """alpha = 1, b = 0: causal linear attention with gated values.

    O = Q S0 + tril(Q K^T) (W*V) and S_T = S0 + K^T (W*V) per (b, h).
    """
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 8, 2, 4, 5
    q, k, v, alpha, b, w, S0 = random_inputs(rng, B, T, H, dk, dv)
    alpha = np.ones_like(alpha)
    b = np.zeros_like(b)
    o, S_T = forward(q, k, v, alpha, b, w, S0)
    for bb in range(B):
        for h in range(H):
            Q, K, U = q[bb, :, h], k[bb, :, h], (w * v)[bb, :, h]
            o_ref = Q @ S0[bb, h] + np.tril(Q @ K.T) @ U
            np.testing.assert_allclose(o[bb, :, h], o_ref, rtol=0, atol=1e-13)
            np.testing.assert_allclose(S_T[bb, h], S0[bb, h] + K.T @ U, rtol=0, atol=1e-13)


def pin_key_value_table(forward, seed=5):
    """One-hot keys e_t (t < d_k), alpha = b = w = 1, S0 = 0: row t of S_T is v_t."""
    rng = np.random.default_rng(seed)
    dk, dv, T = 6, 4, 5
    k = np.zeros((1, T, 1, dk))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    v = rng.standard_normal((1, T, 1, dv))
    ones_k = np.ones((1, T, 1, dk))
    ones_v = np.ones((1, T, 1, dv))
    q = np.zeros((1, T, 1, dk))
    q[0, :, 0, 0] = 1.0  # always look up the first key
    o, S_T = forward(q, k, v, ones_k, ones_k, ones_v, None)
    S_ref = np.zeros((dk, dv))
    S_ref[:T] = v[0, :, 0]
    np.testing.assert_array_equal(S_T[0, 0], S_ref)
    np.testing.assert_array_equal(o[0, :, 0], np.repeat(v[0, :1, 0], T, axis=0))


def pin_overwrite(forward):
    """The same key twice with b = 1, alpha = 1: the second value replaces the first."""
    dk, dv = 3, 2
    k = np.zeros((1, 2, 1, dk))
    k[0, :, 0, 1] = 1.0
    v = np.array([[[[5.0, -1.0]], [[2.0, 7.0]]]])
    w = np.array([[[[1.0, 1.0]], [[0.5, 1.0]]]])
    ones = np.ones((1, 2, 1, dk))
    o, S_T = forward(k, k, v, ones, ones, w, None)
    np.testing.assert_array_equal(o[0, :, 0], np.array([[5.0, -1.0], [1.0, 7.0]]))
    ref = np.zeros((dk, dv))
    ref[1] = [1.0, 7.0]
    np.testing.assert_array_equal(S_T[0, 0], ref)


def gdn_textbook(q, k, v, alpha_s, beta_s, S0):
    """Gated DeltaNet: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.

    Scalar alpha_t, beta_t per (b, t, h); written in the key-by-value state orientation.
    """
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[bb, h].copy()
            for t in range(T):
                kt, a, be = k[bb, t, h], alpha_s[bb, t, h], beta_s[bb, t, h]
                S = a * (S - be * np.outer(kt, kt @ S)) + be * np.outer(kt, v[bb, t, h])
                o[bb, t, h] = S.T @ q[bb, t, h]
            S_T[bb, h] = S
    return o, S_T


def kda_textbook(q, k, v, alpha, beta_s, S0):
    """KDA: S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[bb, h].copy()
            for t in range(T):
                kt, be = k[bb, t, h], beta_s[bb, t, h]
                D = alpha[bb, t, h][:, None] * S
                S = D - be * np.outer(kt, kt @ D) + be * np.outer(kt, v[bb, t, h])
                o[bb, t, h] = S.T @ q[bb, t, h]
            S_T[bb, h] = S
    return o, S_T


def pin_collapse(forward, seed=6):
    """Collapsed gates reproduce KDA, Gated DeltaNet and DeltaNet.

    Page "NVIDIA улучшила память LLM без роста затрат на контекст": the authors state that KDA
    is the case where both gates collapse to one scalar (beta_t of the earlier models) and
    Gated DeltaNet the case where the decay collapses too.
    """
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 10, 2, 5, 4
    q, k, v, alpha, _, _, S0 = random_inputs(rng, B, T, H, dk, dv)
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    a_s = 1 / (1 + np.exp(-(rng.standard_normal((B, T, H)) + 2.0)))
    bk = np.repeat(beta[..., None], dk, axis=-1)
    bv = np.repeat(beta[..., None], dv, axis=-1)
    # KDA: scalar beta, channel-wise alpha
    o, S_T = forward(q, k, v, alpha, bk, bv, S0)
    o_r, S_r = kda_textbook(q, k, v, alpha, beta, S0)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_T, S_r, rtol=0, atol=1e-13)
    # Gated DeltaNet: scalar beta and scalar alpha
    ak = np.repeat(a_s[..., None], dk, axis=-1)
    o, S_T = forward(q, k, v, ak, bk, bv, S0)
    o_r, S_r = gdn_textbook(q, k, v, a_s, beta, S0)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_T, S_r, rtol=0, atol=1e-13)
    # DeltaNet: Gated DeltaNet with alpha = 1
    o, S_T = forward(q, k, v, np.ones_like(ak), bk, bv, S0)
    o_r, S_r = gdn_textbook(q, k, v, np.ones_like(a_s), beta, S0)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_T, S_r, rtol=0, atol=1e-13)


ALL_PINS = [pin_hand_examples, pin_brute_force, pin_exact_write, pin_pure_decay,
            pin_linear_attention, pin_key_value_table, pin_overwrite, pin_collapse]
