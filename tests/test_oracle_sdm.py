"""Pins of the sparse delta memory oracle (``oracle/sdm.py``) against what the pages and the
mathematics fix, and planted mistakes that the pins must catch.

- dense collapse: with N = d_k slots, every slot written and read, write weights k_t and read
  weights q_t, the sparse update is the dense Gated DeltaNet-2 layer with scalar decay and erase
  gates (page "NVIDIA представила Gated DeltaNet-2 ...", "Техническая схема"); checked against
  the C oracle of that layer, which is pinned on its own;
- exact write: one slot at weight 1 with alpha = b = 1 and w = 1 holds exactly v afterwards
  (the delta rule's overwrite), and reading it returns v;
- slots no token writes only decay: M_T[j] = prod(alpha) M0[j];
- pure decay (b = w = 0) and pure accumulation (alpha = 1, b = 0) closed forms;
- a key-value table: one-hot writes of distinct values to distinct slots read back exactly;
- product-key addressing: the two-stage top-m equals the top-m over all n^2 pair sums (brute
  force), weights are the softmax of the chosen sums, W = R = 64 distinct slots
  (aiweekly.co, "Meta FAIR dévoile SDM ...", second paragraph).
"""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import sdm as SDM


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- pins (take an sdm module)

def pin_dense_collapse(m):
    r = _rng(1)
    B, T, H, d = 2, 9, 2, 8
    q, k = _unit(r.standard_normal((B, T, H, d))), _unit(r.standard_normal((B, T, H, d)))
    v = r.standard_normal((B, T, H, d))
    al = r.uniform(0.6, 1.0, (B, T, H))
    be = r.uniform(0.0, 1.0, (B, T, H))
    w = r.uniform(0.0, 1.0, (B, T, H, d))
    M0 = r.standard_normal((B, H, d, d)) * 0.3
    every = np.broadcast_to(np.arange(d), (B, T, H, d))
    o, MT = m.sdm_forward(v, al, be, w, every, k, every, q, M0)
    a_vec = np.repeat(al[..., None], d, axis=-1)
    b_vec = np.repeat(be[..., None], d, axis=-1)
    o_ref, S_ref = oracle.forward(q, k, v, a_vec, b_vec, w, M0, threads=1)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12) and np.allclose(MT, S_ref, rtol=0, atol=1e-12)


def pin_exact_write(m):
    r = _rng(2)
    N, dv = 32, 6
    M = r.standard_normal((N, dv))
    keep = M.copy()
    v = r.standard_normal(dv)
    o = m.sdm_step(M, v, 1.0, 1.0, np.ones(dv), np.array([5]), np.array([1.0]), np.array([5]), np.array([1.0]))
    assert np.allclose(M[5], v, atol=1e-15) and np.allclose(o, v, atol=1e-15)
    others = np.arange(N) != 5
    assert np.array_equal(M[others], keep[others])


def pin_untouched_slots_only_decay(m):
    r = _rng(3)
    B, T, H, N, dv, W = 1, 7, 1, 24, 4, 3
    v = r.standard_normal((B, T, H, dv))
    al = r.uniform(0.5, 1.0, (B, T, H))
    be = r.uniform(0.0, 1.0, (B, T, H))
    widx = np.stack([r.choice(12, W, replace=False) for _ in range(T)]).reshape(B, T, H, W)  # slots 0..11 only
    wwt = r.dirichlet(np.ones(W), size=(B, T, H))
    ridx = r.integers(0, N, (B, T, H, 1))
    M0 = r.standard_normal((B, H, N, dv))
    _, MT = m.sdm_forward(v, al, be, None, widx, wwt, ridx, np.ones((B, T, H, 1)), M0)
    assert np.allclose(MT[0, 0, 12:], np.prod(al) * M0[0, 0, 12:], rtol=1e-13, atol=0)


def pin_pure_decay(m):
    r = _rng(4)
    B, T, H, N, dv, W, R = 1, 6, 2, 20, 5, 4, 3
    v = r.standard_normal((B, T, H, dv))
    al = r.uniform(0.5, 1.0, (B, T, H))
    widx = np.stack([r.choice(N, W, replace=False) for _ in range(B * T * H)]).reshape(B, T, H, W)
    ridx = np.stack([r.choice(N, R, replace=False) for _ in range(B * T * H)]).reshape(B, T, H, R)
    wwt, rwt = r.dirichlet(np.ones(W), size=(B, T, H)), r.dirichlet(np.ones(R), size=(B, T, H))
    M0 = r.standard_normal((B, H, N, dv))
    o, MT = m.sdm_forward(v, al, np.zeros((B, T, H)), np.zeros((B, T, H, dv)), widx, wwt, ridx, rwt, M0)
    g = np.cumprod(al, axis=1)  # [B, T, H]
    for h in range(H):
        assert np.allclose(MT[0, h], g[0, -1, h] * M0[0, h], rtol=1e-13, atol=0)
        for t in range(T):
            want = g[0, t, h] * (rwt[0, t, h] @ M0[0, h][ridx[0, t, h]])
            assert np.allclose(o[0, t, h], want, rtol=1e-12, atol=1e-14)


def pin_pure_accumulation(m):
    r = _rng(5)
    B, T, H, N, dv, W = 1, 8, 1, 16, 3, 4
    v = r.standard_normal((B, T, H, dv))
    w = r.uniform(0, 1, (B, T, H, dv))
    widx = np.stack([r.choice(N, W, replace=False) for _ in range(T)]).reshape(B, T, H, W)
    wwt = r.dirichlet(np.ones(W), size=(B, T, H))
    M0 = r.standard_normal((B, H, N, dv))
    _, MT = m.sdm_forward(v, np.ones((B, T, H)), np.zeros((B, T, H)), w, widx, wwt, widx, wwt, M0)
    want = M0[0, 0].copy()
    for t in range(T):  # sum of scattered outer products a_t (w_t * v_t)^T
        for s, a in zip(widx[0, t, 0], wwt[0, t, 0]):
            want[s] += a * w[0, t, 0] * v[0, t, 0]
    assert np.allclose(MT[0, 0], want, rtol=1e-13, atol=1e-14)


def pin_key_value_table(m):
    r = _rng(6)
    N, dv = 10, 4
    vals = r.standard_normal((N, dv))
    T = N
    order = r.permutation(N)
    v = vals[order].reshape(1, T, 1, dv)
    one = np.ones((1, T, 1))
    widx = order.reshape(1, T, 1, 1)
    M0 = r.standard_normal((1, 1, N, dv))  # overwritten slot by slot
    o, MT = m.sdm_forward(v, one, one, None, widx, np.ones((1, T, 1, 1)), widx, np.ones((1, T, 1, 1)), M0)
    assert np.allclose(MT[0, 0], vals, atol=1e-14) and np.allclose(o[0, :, 0], vals[order], atol=1e-14)


def pin_pkm_brute_force(m):
    r = _rng(7)
    for n, half, mm, Q in ((16, 4, 5, 40), (64, 8, 64, 6), (8, 2, 8, 10), (12, 3, 1, 10)):
        C1, C2 = r.standard_normal((n, half)), r.standard_normal((n, half))
        x = r.standard_normal((Q, 2 * half))
        idx, wt = m.pkm_address(x, C1, C2, mm)
        assert idx.shape == (Q, mm) and wt.shape == (Q, mm)
        for qi in range(Q):
            full = (C1 @ x[qi, :half])[:, None] + (C2 @ x[qi, half:])[None, :]  # all n^2 pair sums
            flat = full.ravel()                                                 # slot i * n + j
            top = np.argsort(-flat, kind="stable")[:mm]
            assert np.array_equal(idx[qi], top)
            e = np.exp(flat[top] - flat[top].max())
            assert np.allclose(wt[qi], e / e.sum(), rtol=1e-13, atol=0)
            assert len(set(idx[qi])) == mm and idx[qi].max() < n * n
        assert np.allclose(wt.sum(-1), 1.0, atol=1e-14)


PINS = [pin_dense_collapse, pin_exact_write, pin_untouched_slots_only_decay, pin_pure_decay,
        pin_pure_accumulation, pin_key_value_table, pin_pkm_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(SDM)


def test_w_r_64_slots_of_n():
    """W = R = 64 slots of N = 256^2 per token (d_k = 128: two halves of 64)."""
    r = _rng(8)
    n, dk = 256, 128
    C1, C2 = r.standard_normal((n, dk // 2)) / 8, r.standard_normal((n, dk // 2)) / 8
    x = _unit(r.standard_normal((3, dk)))
    idx, wt = oracle.pkm_address(x, C1, C2, 64)
    assert idx.shape == (3, 64)
    for row in idx:
        assert len(set(row.tolist())) == 64 and row.min() >= 0 and row.max() < n * n
    assert np.allclose(wt.sum(-1), 1.0)


def test_duplicate_write_slots_rejected():
    with pytest.raises(ValueError):
        SDM.sdm_step(np.zeros((4, 2)), np.ones(2), 1.0, 1.0, np.ones(2), np.array([1, 1]), np.ones(2) / 2,
                     np.array([0]), np.ones(1))


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "decay_dropped": ("M *= alpha  ", "M *= 1.0  "),
    "decay_only_on_written_slots": ("M *= alpha  ", "M[widx] *= alpha  "),
    "erase_reads_undecayed": ("e = wwt @ M[widx]", "e = wwt @ M[widx] / alpha"),
    "erase_sign_flipped": ("(w * v - b * e)", "(w * v + b * e)"),
    "erase_gate_dropped": ("(w * v - b * e)", "(w * v - e)"),
    "write_gate_dropped": ("(w * v - b * e)", "(v - b * e)"),
    "write_weight_dropped": ("M[widx] += wwt[:, None] * ", "M[widx] += "),
    "read_slots_misaligned": ("return rwt @ M[ridx]", "return rwt @ M[ridx[::-1]]"),
    "pkm_second_half_reads_first": ("s2 = C2 @ xq[half:]", "s2 = C2 @ xq[:half]"),
    "pkm_slot_index_transposed": ("slot = (I[:, None] * n + J[None, :]).ravel()",
                                  "slot = (J[None, :] * n + I[:, None]).ravel()"),
    "pkm_too_few_candidates": ("I = np.lexsort((np.arange(n), -s1))[:m]",
                               "I = np.lexsort((np.arange(n), -s1))[:max(1, m // 2)]"),
    "pkm_weights_unnormalised": ("wt[r] = e / e.sum()", "wt[r] = e"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SDM.__file__).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType("sdm_mutant_" + name)
    exec(compile(src.replace(old, new), os.path.join("mutant", name + ".py"), "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the mutant {name}"
