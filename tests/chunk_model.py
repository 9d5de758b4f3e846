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


def _split_bf16(x):
    hi = round_bf16(x)
    return hi, round_bf16(round_f32(x - hi))


def _mm16(a, b):
    """fp16 operands, fp32 result (one matrix-core pass)."""
    return round_f32(round_f16(a) @ round_f16(b))


def _mm_bf16x3(a, b):
    """bf16 hi/lo split operands, hi*hi + hi*lo + lo*hi, fp32 result."""
    ah, al = _split_bf16(a)
    bh, bl = _split_bf16(b)
    return round_f32(ah @ bh + ah @ bl + al @ bh)


def kernel_scheme_model(q, k, v, alpha, b, w, S0=None, *, delta_form="TU-WS", diag="bf16x3"):
    """The chunk kernel's exact operand-precision scheme for bf16 inputs, in numpy.

    delta_form "TU-WS" forms W = T E_hat and U~ = T U first; "T(U-ES)" applies T after
    subtracting E_hat S (no W). diag "bf16x3" or "f16" selects the diagonal Gram operands.

    C = 64 in four 16-row blocks. Vector math in fp32. Gram blocks below the diagonal: fp16
    operands with block-boundary references (row side exp(local), times exp(G_I - G_{J+1})
    when blocks are not adjacent; column side exp(blocktot_J - local)). Diagonal Gram blocks:
    bf16 hi/lo split operands (three passes) with the block's 8th row as reference, so no
    factor exceeds the decay of 8 tokens. UT inverse: 16x16 diagonal blocks by fp32 forward
    substitution, merged at 32 and 64 rows by fp16 products. W, U~ and the state-chain
    products take fp16 operands with fp32 results; the state stays fp32.
    """
    q, k, v, alpha, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, b, w))
    T_len, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else round_f32(np.array(S0, dtype=np.float64))
    o = np.zeros((T_len, dv))
    C = 64
    for c0 in range(0, T_len, C):
        L = min(C, T_len - c0)
        pad = C - L

        def P_(x, fill):
            x = x[c0:c0 + L]
            return np.concatenate([x, np.full((pad, x.shape[1]), fill)]) if pad else x
        qc, kc, bc = P_(q, 0.0), P_(k, 0.0), P_(b, 0.0)
        ac = P_(alpha, 1.0)
        vc, wc = P_(v, 0.0), P_(w, 0.0)
        g = round_f32(np.log(ac))
        local = np.zeros_like(g)
        for blk in range(4):
            run = np.zeros(dk)
            for r in range(16 * blk, 16 * blk + 16):
                run = round_f32(run + g[r])
                local[r] = run
        tot = local[15::16]  # [4, dk] block totals
        G = np.zeros((5, dk))
        for n in range(1, 5):
            G[n] = round_f32(G[n - 1] + tot[n - 1])
        Gam = round_f32(np.repeat(G[:4], 16, axis=0) + local)
        e = round_f32(bc * kc)
        A = np.zeros((C, C))
        Pm = np.zeros((C, C))
        for I in range(4):
            rI = slice(16 * I, 16 * I + 16)
            fr = round_f32(np.exp(local[rI]))
            e_ref = round_f32(e[rI] * fr)
            q_ref = round_f32(qc[rI] * fr)
            X = local[16 * I + 7]
            fm = round_f32(np.exp(round_f32(local[rI] - X)))
            km = round_f32(kc[rI] * round_f32(np.exp(round_f32(X - local[rI]))))
            mm_diag = _mm_bf16x3 if diag == "bf16x3" else _mm16
            A[rI, rI] = mm_diag(round_f32(e[rI] * fm), km.T)
            Pm[rI, rI] = mm_diag(round_f32(qc[rI] * fm), km.T)
            for J in range(I):
                rJ = slice(16 * J, 16 * J + 16)
                kt = round_f32(kc[rJ] * round_f32(np.exp(round_f32(tot[J] - local[rJ]))))
                cIJ = round_f32(np.exp(round_f32(G[I] - G[J + 1])))
                A[rI, rJ] = _mm16(round_f32(e_ref * cIJ), kt.T)
                Pm[rI, rJ] = _mm16(round_f32(q_ref * cIJ), kt.T)
        A = np.tril(A, -1)
        Pm = np.tril(Pm, 0)
        # UT inverse
        Tm = np.zeros((C, C))
        for I in range(4):
            rI = slice(16 * I, 16 * I + 16)
            a = A[rI, rI]
            t = np.zeros((16, 16))
            for r in range(16):
                t[r, r] = 1.0
                if r:
                    t[r, :r] = round_f32(-(a[r, :r] @ t[:r, :r]))
            Tm[rI, rI] = t
        for I, J in ((1, 0), (3, 2)):
            rI, rJ = slice(16 * I, 16 * I + 16), slice(16 * J, 16 * J + 16)
            X = _mm16(A[rI, rJ], Tm[rJ, rJ])
            Tm[rI, rJ] = -_mm16(Tm[rI, rI], X)
        Y = _mm16(A[32:, :32], Tm[:32, :32])
        Tm[32:, :32] = -_mm16(Tm[32:, 32:], Y)
        gam = round_f32(np.exp(Gam))
        E_hat = round_f32(e * gam)
        U = round_f32(wc * vc)
        Q_hat = round_f32(qc * gam)
        if delta_form == "TU-WS":
            W = _mm16(Tm, E_hat)
            Ut = _mm16(Tm, U)
            Delta = round_f32(Ut - _mm16(W, S))
        else:  # Delta = T (U - E_hat S)
            Delta = _mm16(Tm, round_f32(U - _mm16(E_hat, S)))
        O = round_f32(_mm16(Q_hat, S) + _mm16(Pm, Delta))
        o[c0:c0 + L] = O[:L]
        K_bar = round_f32(kc * round_f32(np.exp(round_f32(Gam[C - 1] - Gam))))
        S = round_f32(gam[C - 1][:, None] * S + _mm16(K_bar.T, Delta))
    return o, S
