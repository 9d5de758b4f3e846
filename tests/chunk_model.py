"""numpy model of the chunkwise (WY / UT) form of the Gated DeltaNet-2 recurrence.

Test infrastructure: it pins the chunk algebra the HIP kernel follows against the
sequential oracle (in float64), and, with operand rounding switched on, emulates the
precision of the kernel's matrix-core products. It shares no code with the HIP path.

Chunking with C = 64 and the cumulative channel-wise decay absorbed into the rank-1 factors
follow the page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph
"Реализация". The algebra, for a chunk of rows r = 1..L with incoming state S:

    Gamma_r = sum_{s<=r} log alpha_s,  gamma_r = exp(Gamma_r)            (per key channel)
    e_hat_r = gamma_r*b_r*k_r,  k_hat_j = k_j/gamma_j,  q_hat_r = gamma_r*q_r
    A = strictLower(E_hat K_hat^T),  P = lowerIncl(Q_hat K_hat^T)         (Gram products)
    T = (I + A)^-1,  W = T E_hat,  U~ = T (w*v)                            (UT transform)
    Delta = U~ - W S,  O = Q_hat S + P Delta,  S <- Diag(gamma_L) S + K_bar^T Delta
    with k_bar_j = (gamma_L/gamma_j)*k_j.

The Gram products are formed per 16x16 block with reference points so every factor stays
bounded: for a block (I, J) below the diagonal the row factor is scaled by exp(Gamma_r - G_I),
the column factor by exp(G_{J+1} - Gamma_j) and their product by exp(G_I - G_{J+1}), where
G_n is Gamma at the last row before block n (each factor <= 1); diagonal blocks use the
block's start as reference.
"""
from __future__ import annotations

import numpy as np

BLK = 16


def round_bf16(x):
    """Round to bfloat16 (nearest-even) and return as float64."""
    x32 = np.asarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def make_operand_rounder(kind):
    """Return f(x) -> list of (part) arrays whose sum approximates x, as a product operand.

    kind: "f64" exact; "f32"; "bf16"/"f16" one rounded part; "bf16x2"/"f16x2" hi + lo parts.
    """
    if kind == "f64":
        return lambda x: [_ident(x)]
    if kind == "f32":
        return lambda x: [round_f32(x)]
    base = {"bf16": round_bf16, "f16": round_f16}[kind.split("x")[0]]
    if kind.endswith("x2"):
        def split(x):
            x = round_f32(x)
            hi = base(x)
            return [hi, base(x - hi)]
        return split
    return lambda x: [base(x)]


def product(a, b, ka="f64", kb="f64", acc="f64", drop_lo_lo=True):
    """Emulated matrix-core product a @ b: operands split/rounded, fp32 (or f64) result."""
    pa = make_operand_rounder(ka)(a)
    pb = make_operand_rounder(kb)(b)
    out = np.zeros((np.shape(a)[0], np.shape(b)[1]))
    for i, x in enumerate(pa):
        for j, y in enumerate(pb):
            if drop_lo_lo and i > 0 and j > 0:
                continue
            out = out + x @ y
    return round_f32(out) if acc == "f32" else out


DEFAULT_PREC = dict(gram="f64", ut="f64", wu="f64", state="f64", out="f64", carry="f64",
                    s_op="f64", fp32_vector=False)


def chunk_forward_model(q, k, v, alpha, b, w, S0=None, *, C=64, prec=None):
    """One sequence: q, k, alpha, b [T, d_k]; v, w [T, d_v]; S0 [d_k, d_v] or None.

    prec maps product groups to operand kinds (see make_operand_rounder):
      gram  - A and P Gram products          ut - (unused: the UT solve is f32/f64 vector math)
      wu    - W = T E_hat and U~ = T U        state - W S and Q_hat S (the non-state operand)
      s_op  - the state operand of W S, Q_hat S
      out   - P Delta                          carry - K_bar^T Delta
      fp32_vector - do the vector math (logs, cumsums, exps, solve, state scaling) in fp32
    Returns (o [T, d_v], S_T [d_k, d_v]) in float64.
    """
    p = dict(DEFAULT_PREC)
    if prec:
        p.update(prec)
    acc = "f32" if p["fp32_vector"] else "f64"
    vr = round_f32 if p["fp32_vector"] else _ident
    q, k, v, alpha, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, b, w))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        sl = slice(c0, c0 + L)
        qc, kc, vc, ac, bc, wc = q[sl], k[sl], v[sl], alpha[sl], b[sl], w[sl]
        # gate prep: log-decay and its inclusive cumulative sum over the chunk's rows
        g = vr(np.log(ac))
        Gam = np.zeros_like(g)
        run = np.zeros(dk)
        for r in range(L):
            run = vr(run + g[r])
            Gam[r] = run
        gam = vr(np.exp(Gam))
        e = vr(bc * kc)
        # Gram products with block reference points
        nb = (L + BLK - 1) // BLK
        Gref = np.zeros((nb + 1, dk))  # Gref[n] = Gamma at the last row before block n
        for n in range(1, nb + 1):
            Gref[n] = Gam[min(n * BLK, L) - 1]
        A = np.zeros((L, L))
        Pm = np.zeros((L, L))
        for I in range(nb):
            rI = slice(I * BLK, min((I + 1) * BLK, L))
            e_I = vr(e[rI] * vr(np.exp(vr(Gam[rI] - Gref[I]))))
            q_I = vr(qc[rI] * vr(np.exp(vr(Gam[rI] - Gref[I]))))
            for J in range(I + 1):
                rJ = slice(J * BLK, min((J + 1) * BLK, L))
                if J < I:
                    kt = vr(kc[rJ] * vr(np.exp(vr(Gref[J + 1] - Gam[rJ]))))
                    kt = vr(kt * vr(np.exp(vr(Gref[I] - Gref[J + 1]))))
                else:
                    kt = vr(kc[rJ] * vr(np.exp(vr(Gref[I] - Gam[rJ]))))
                A[rI, rJ] = product(e_I, kt.T, p["gram"], p["gram"], acc)
                Pm[rI, rJ] = product(q_I, kt.T, p["gram"], p["gram"], acc)
        A = np.tril(A, -1)
        Pm = np.tril(Pm, 0)
        # UT transform: T = (I + A)^-1 by forward substitution (vector math)
        Tm = np.zeros((L, L))
        for r in range(L):
            row = np.zeros(L)
            row[r] = 1.0
            if r:
                row[:r] = vr(-(A[r, :r] @ Tm[:r, :r]))
            Tm[r] = row
        E_hat = vr(e * gam)
        U = vr(wc * vc)
        W = product(Tm, E_hat, p["wu"], p["wu"], acc)
        Ut = product(Tm, U, p["wu"], p["wu"], acc)
        # state-dependent part
        Q_hat = vr(qc * gam)
        WS = product(W, S, p["state"], p["s_op"], acc)
        Delta = vr(Ut - WS)
        QS = product(Q_hat, S, p["state"], p["s_op"], acc)
        PD = product(Pm, Delta, p["out"], p["out"], acc)
        o[sl] = vr(QS + PD)
        K_bar = vr(kc * vr(np.exp(vr(Gam[L - 1] - Gam))))
        S = vr(gam[L - 1][:, None] * S + product(K_bar.T, Delta, p["carry"], p["carry"], acc))
    return o, S
