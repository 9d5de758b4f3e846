"""fp64 CPU oracle for Sparse Delta Memory (SDM) on the Gated DeltaNet-2 update.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg may import it.

Sources: the aiweekly.co article "Meta FAIR dévoile SDM, un RNN linéaire à mémoire sparse
massive", second paragraph (SDM starts from Gated DeltaNet and replaces the dense key-value outer
product with sparse reads and writes into a large explicit memory; a Product-Key-Memory style
index picks W write and R read slots out of N per token, W = R = 64), its third paragraph (a
learned initial memory M0) and fourth (memory per layer grows as O(d^3)); the gonzo_ML digest
"Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity", TL;DR (state three
orders of magnitude larger at the same FLOPs per token). The update it sparsifies is the page
"NVIDIA представила Gated DeltaNet-2 ...", paragraph "Техническая схема":
S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T.

The pages leave the following open; this oracle takes these readings:
- the memory of one (batch, head) is M in R^{N x d_v}: N slots of d_v values (slots stand where
  the d_k key rows of the dense state stood);
- addressing is product-key top-m (m = W for the write, m = R for the read): the query (k_t for
  the write, q_t for the read) is cut into two halves, each scored against its own table of n
  sub-keys; the m best sub-keys of each half are kept, the m best of their m x m pair sums are
  the slots (slot = i * n + j for sub-keys i and j, N = n^2), and the weights are the softmax of
  those m sums;
- the update is the Gated DeltaNet-2 rule with the key k_t replaced by the N-vector a_t of write
  weights (zero off the W chosen slots). The decay and erase gates act on the key axis, which is
  now the slot axis; they are taken as per-token scalars alpha_t and b_t (a gate per slot is not
  something a token could produce). The write gate acts on the value axis and is kept as the
  d_v-vector w_t:
      M_t = (I - b_t a_t a_t^T) alpha_t M_{t-1} + a_t (w_t * v_t)^T;
  the decay reaches every slot, touched or not (as the dense decay reaches every key row);
- the read is o_t = M_t^T r_t with r_t the N-vector of read weights (zero off the R chosen
  slots), from the updated memory, as the dense layer reads o_t = S_t^T q_t.
With N = d_k, every slot chosen, a_t = k_t and r_t = q_t, the update and read are the dense
Gated DeltaNet-2 layer with scalar alpha and b.

Pinned by ``tests/test_oracle_sdm.py``: the dense special case against the Gated DeltaNet-2
oracle, the sparse update against its dense N x N matrix form, exact write, untouched-slot decay,
pure decay, product-key selection against brute force over all N pair sums, and planted mistakes.
"""
from __future__ import annotations

import numpy as np


def pkm_address(x, C1, C2, m: int):
    """Product-key top-m addressing of queries x [..., d_k] over N = n^2 slots, float64.

    C1, C2: sub-key tables [n, d_k / 2] for the first and second half of the query.
    Returns (idx [..., m] int64, weight [..., m] float64): the chosen slots i * n + j, best pair
    sum first (equal sums: lower slot first), and the softmax of their sums.
    """
    x = np.asarray(x, dtype=np.float64)
    C1 = np.asarray(C1, dtype=np.float64)
    C2 = np.asarray(C2, dtype=np.float64)
    n, half = C1.shape
    if C2.shape != (n, half) or x.shape[-1] != 2 * half:
        raise ValueError("sub-key tables must be [n, d_k/2] each, queries [..., d_k]")
    if not 1 <= m <= n:
        raise ValueError("m must be in [1, n]")
    lead = x.shape[:-1]
    xs = x.reshape(-1, 2 * half)
    idx = np.empty((xs.shape[0], m), dtype=np.int64)
    wt = np.empty((xs.shape[0], m), dtype=np.float64)
    for r, xq in enumerate(xs):
        s1 = C1 @ xq[:half]
        s2 = C2 @ xq[half:]
        # m best sub-keys of each half (equal scores: lower index first)
        I = np.lexsort((np.arange(n), -s1))[:m]
        J = np.lexsort((np.arange(n), -s2))[:m]
        pair = (s1[I][:, None] + s2[J][None, :]).ravel()
        slot = (I[:, None] * n + J[None, :]).ravel()
        best = np.lexsort((slot, -pair))[:m]
        sc = pair[best]
        e = np.exp(sc - sc.max())
        idx[r] = slot[best]
        wt[r] = e / e.sum()
    return idx.reshape(*lead, m), wt.reshape(*lead, m)


def sdm_step(M, v, alpha, b, w, widx, wwt, ridx, rwt):
    """One token of one (batch, head): the memory M [N, d_v] (float64, updated in place) and the
    read o [d_v] it returns.

    widx/wwt: the W write slots (distinct) and their weights; ridx/rwt: the R read slots and
    weights; alpha, b: scalars; v, w: [d_v].
    """
    widx = np.asarray(widx)
    if len(np.unique(widx)) != len(widx):
        raise ValueError("write slots must be distinct")
    M *= alpha                                  # Diag(alpha) on every slot
    e = wwt @ M[widx]                           # a^T (alpha M): what the write slots hold
    M[widx] += wwt[:, None] * (w * v - b * e)[None, :]  # - b a a^T (alpha M) + a (w * v)^T
    return rwt @ M[ridx]                        # o = M^T r


def sdm_forward(v, alpha, b, w, widx, wwt, ridx, rwt, M0=None, *, N: int | None = None):
    """Sparse delta memory over [B, T, H, ...] inputs in float64.

    v, w: [B, T, H, d_v] (w None: all ones); alpha, b: [B, T, H];
    widx, wwt: [B, T, H, W]; ridx, rwt: [B, T, H, R]; M0: [B, H, N, d_v] or None (zeros, then N
    must be given). Returns (o [B, T, H, d_v], M_T [B, H, N, d_v]).
    """
    v = np.asarray(v, dtype=np.float64)
    B, T, H, dv = v.shape
    alpha = np.asarray(alpha, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    w = np.ones_like(v) if w is None else np.asarray(w, dtype=np.float64)
    wwt = np.asarray(wwt, dtype=np.float64)
    rwt = np.asarray(rwt, dtype=np.float64)
    if M0 is None:
        if N is None:
            raise ValueError("N is needed when M0 is None")
        M = np.zeros((B, H, N, dv))
    else:
        M = np.array(M0, dtype=np.float64, copy=True)
    o = np.empty((B, T, H, dv))
    for bb in range(B):
        for hh in range(H):
            Mh = M[bb, hh]
            for t in range(T):
                o[bb, t, hh] = sdm_step(Mh, v[bb, t, hh], alpha[bb, t, hh], b[bb, t, hh], w[bb, t, hh],
                                        widx[bb, t, hh], wwt[bb, t, hh], ridx[bb, t, hh], rwt[bb, t, hh])
    return o, M
