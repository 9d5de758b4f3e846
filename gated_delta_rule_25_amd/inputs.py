"""Seeded synthetic inputs for the Gated DeltaNet-2 prefill and decode workloads.

This module only draws and shapes random numbers; it holds none of the recurrence's
arithmetic. Both the HIP path's tests and the oracle's tests take their inputs from here.

Distributions follow the layer the pages describe: q and k pass through an L2 norm per head
and the gates are sigmoids of token projections (page "NVIDIA представила Gated DeltaNet-2 с
канал-wise гейтами …", paragraphs "Техническая схема" and "Архитектурно"); the state is
262,144 floats per layer per batch element, i.e. 16 heads of 128x128 (page "NVIDIA улучшила
память LLM без роста затрат на контекст", section "Аналитика"). Since no trained projections
exist here, the pre-activations are standard normals:

    q, k  = L2normalize(N(0,1)) over d_k          v = N(0,1)
    b, w  = sigmoid(N(0,1)) per channel           alpha = sigmoid(N(alpha_mu, 1)) per key channel
    S0    = N(0, s0_std^2) (or zero)              beta (scalar gates) = sigmoid(N(0,1)) per token

Draw order (numpy backend): q, k, v, b, w, alpha, S0, then beta. Values are drawn in float32
and rounded to bfloat16 with round-to-nearest-even when dtype is bf16; the same rounded
tensors go to the GPU and to the oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named input recipe (shapes, dtype and distributions)."""
    name: str
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    dtype: str = "bf16"  # "bf16" or "fp32": dtype of q, k, v, alpha, b, w
    alpha_mu: float = 3.0
    s0_std: float = 0.1  # 0 => zero initial state
    gates: str = "general"  # "general", "gdn" (scalar alpha and beta), "kda" (scalar beta)
    seed: int = 20250


# Named workloads. Sizes follow the pages' 1.3B setting (16 heads of 128x128).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, T=256, H=2, d_k=32, d_v=32, dtype="fp32",
                          s0_std=0.0, seed=20250),
    "prefill_1p3b": Workload("prefill_1p3b", B=8, T=4096, H=16, d_k=128, d_v=128, seed=20251),
    "long_prefill": Workload("long_prefill", B=1, T=131072, H=16, d_k=128, d_v=128,
                             alpha_mu=5.0, seed=20252),
    "gdn_scalar": Workload("gdn_scalar", B=8, T=4096, H=16, d_k=128, d_v=128, gates="gdn",
                           seed=20253),
    "kda_scalar": Workload("kda_scalar", B=8, T=4096, H=16, d_k=128, d_v=128, gates="kda",
                           seed=20253),
    # head size 256 with the same 262,144 state floats per batch element (4 heads of 256 x 256)
    "d256_prefill": Workload("d256_prefill", B=8, T=4096, H=4, d_k=256, d_v=256, seed=20262),
    # the 1.3B layer's shape with fp32 inputs (fp32 operands throughout)
    "fp32_prefill": Workload("fp32_prefill", B=8, T=4096, H=16, d_k=128, d_v=128, dtype="fp32", seed=20263),
}

DECODE_WORKLOAD = dict(B=256, H=16, d_k=128, d_v=128, steps=1000, alpha_mu=3.0, s0_std=0.1,
                       seed=20254)


def scaled(wl: Workload, **changes) -> Workload:
    """The same recipe at other sizes (e.g. fewer tokens for a test)."""
    return dataclasses.replace(wl, **changes)


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-12)).astype(np.float32)


def make_inputs(wl: Workload, *, device: str = "cpu") -> dict:
    """Draw one workload's inputs.

    Returns a dict of torch tensors on `device`: q, k, alpha, b [B, T, H, d_k];
    v, w [B, T, H, d_v]; S0 [B, H, d_k, d_v] float32 or None. With scalar gates,
    alpha is [B, T, H] for "gdn", b holds beta as [B, T, H] and w is None; the keys
    "alpha_scalar" and "beta_scalar" say which. Generation uses numpy's PCG64 on the host.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.d_k, wl.d_v
    f32 = np.float32
    q = _l2n(rng.standard_normal((B, T, H, dk), dtype=f32))
    k = _l2n(rng.standard_normal((B, T, H, dk), dtype=f32))
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    b = _sigmoid(rng.standard_normal((B, T, H, dk), dtype=f32))
    w = _sigmoid(rng.standard_normal((B, T, H, dv), dtype=f32))
    a_shape = (B, T, H) if wl.gates == "gdn" else (B, T, H, dk)
    alpha = _sigmoid(rng.standard_normal(a_shape, dtype=f32) + f32(wl.alpha_mu))
    S0 = None
    if wl.s0_std > 0:
        S0 = rng.standard_normal((B, H, dk, dv), dtype=f32) * f32(wl.s0_std)
    beta_scalar = wl.gates in ("gdn", "kda")
    if beta_scalar:
        b = _sigmoid(rng.standard_normal((B, T, H), dtype=f32))
        w = None
    dt = _torch_dtype(wl.dtype)

    def t(x):
        return None if x is None else torch.from_numpy(x).to(dt).to(device)

    return dict(q=t(q), k=t(k), v=t(v), alpha=t(alpha), b=t(b), w=t(w),
                S0=None if S0 is None else torch.from_numpy(S0).to(device),
                alpha_scalar=(wl.gates == "gdn"), beta_scalar=beta_scalar)


def make_prologue_inputs(wl: Workload, *, device: str = "cpu") -> dict:
    """Raw inputs for the fused prologue (in-kernel L2 norm and gate logits): q, k standard normal
    times a per-token scale drawn uniformly from [0.5, 4] (so the norm matters), v standard
    normal, and the gates as pre-activations: alpha ~ N(alpha_mu, 1), b, w ~ N(0, 1) (scalar
    forms as in make_inputs). Same dict layout as make_inputs; drawn from seed + 104729."""
    rng = np.random.Generator(np.random.PCG64(wl.seed + 104729))
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.d_k, wl.d_v
    f32 = np.float32
    q = rng.standard_normal((B, T, H, dk), dtype=f32) * rng.uniform(0.5, 4.0, (B, T, H, 1)).astype(f32)
    k = rng.standard_normal((B, T, H, dk), dtype=f32) * rng.uniform(0.5, 4.0, (B, T, H, 1)).astype(f32)
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    b = rng.standard_normal((B, T, H, dk), dtype=f32)
    w = rng.standard_normal((B, T, H, dv), dtype=f32)
    a_shape = (B, T, H) if wl.gates == "gdn" else (B, T, H, dk)
    alpha = rng.standard_normal(a_shape, dtype=f32) + f32(wl.alpha_mu)
    S0 = rng.standard_normal((B, H, dk, dv), dtype=f32) * f32(wl.s0_std) if wl.s0_std > 0 else None
    beta_scalar = wl.gates in ("gdn", "kda")
    if beta_scalar:
        b = rng.standard_normal((B, T, H), dtype=f32)
        w = None
    dt = _torch_dtype(wl.dtype)

    def t(x):
        return None if x is None else torch.from_numpy(x).to(dt).to(device)

    return dict(q=t(q), k=t(k), v=t(v), alpha=t(alpha), b=t(b), w=t(w),
                S0=None if S0 is None else torch.from_numpy(S0).to(device),
                alpha_scalar=(wl.gates == "gdn"), beta_scalar=beta_scalar)


def packed_lengths(n: int, total: int, *, seed: int, lo: int = 16, hi: int = 4096) -> list:
    """A length mix for a packed batch: n lengths drawn log-uniformly in [lo, hi], rescaled to sum
    to `total` (floored; the remainder goes to the last sequence). Serving batches mix short and
    long prompts; the pages give no length distribution, so this one is a stand-in."""
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = np.exp(rng.uniform(np.log(lo), np.log(hi), n))
    ls = np.floor(raw / raw.sum() * total).astype(np.int64)
    ls[-1] += total - int(ls.sum())
    return [int(x) for x in ls]


def make_packed_inputs(wl: Workload, lengths, *, device: str = "cpu", raw: bool = False) -> dict:
    """A packed batch of len(lengths) sequences: the workload's recipe drawn as one row of
    sum(lengths) tokens (B = 1, then the batch axis dropped: q [T_total, H, d_k] ...), one
    initial state per sequence ([N, H, d_k, d_v], seed + 15485863, or None when s0_std is 0) and
    cu_seqlens [N + 1] int32. raw=True draws the prologue recipe (make_prologue_inputs)."""
    T = int(sum(lengths))
    one = dataclasses.replace(wl, B=1, T=T)
    ins = (make_prologue_inputs if raw else make_inputs)(one, device="cpu")
    for n in ("q", "k", "v", "alpha", "b", "w"):
        if ins[n] is not None:
            ins[n] = ins[n][0].contiguous().to(device)
    N = len(lengths)
    rng = np.random.Generator(np.random.PCG64(wl.seed + 15485863))
    S0 = None
    if wl.s0_std > 0:
        S0 = torch.from_numpy(rng.standard_normal((N, wl.H, wl.d_k, wl.d_v), dtype=np.float32)
                              * np.float32(wl.s0_std)).to(device)
    ins["S0"] = S0
    ins["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to(device)
    return ins


def make_cotangents(wl: Workload, *, device: str = "cpu", final_state: bool = True) -> dict:
    """Seeded cotangents for the backward: dO [B, T, H, d_v] and dS_T [B, H, d_k, d_v] (or None),
    both standard normal in float32, drawn from their own stream (seed + 7919)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed + 7919))
    f32 = np.float32
    dO = rng.standard_normal((wl.B, wl.T, wl.H, wl.d_v), dtype=f32)
    dS = rng.standard_normal((wl.B, wl.H, wl.d_k, wl.d_v), dtype=f32) if final_state else None
    return dict(dO=torch.from_numpy(dO).to(device),
                dS_T=None if dS is None else torch.from_numpy(dS).to(device))


def make_packed_cotangents(wl: Workload, lengths, *, device: str = "cpu", final_state: bool = True) -> dict:
    """Cotangents for a packed batch (make_packed_inputs): dO [sum(lengths), H, d_v] and dS_T
    [N, H, d_k, d_v] (or None), standard normal float32 from their own stream (seed + 7919)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed + 7919))
    f32 = np.float32
    dO = rng.standard_normal((int(sum(lengths)), wl.H, wl.d_v), dtype=f32)
    dS = rng.standard_normal((len(lengths), wl.H, wl.d_k, wl.d_v), dtype=f32) if final_state else None
    return dict(dO=torch.from_numpy(dO).to(device),
                dS_T=None if dS is None else torch.from_numpy(dS).to(device))


def make_decode_inputs(B: int, H: int, d_k: int, d_v: int, steps: int, *, seed: int,
                       alpha_mu: float = 3.0, s0_std: float = 0.1, dtype: str = "bf16",
                       device: str = "cpu", generator: str = "numpy") -> dict:
    """Inputs for `steps` consecutive single-token steps.

    Returns q, k, alpha, b [steps, B, H, d_k]; v, w [steps, B, H, d_v]; S0 [B, H, d_k, d_v].
    generator="numpy" draws on the host (PCG64, as make_inputs); generator="torch" draws with
    a seeded torch.Generator on `device` (Philox on a GPU), which is much faster for the
    thousand-step decode workload. Both are deterministic for a given seed.
    """
    dt = _torch_dtype(dtype)
    if generator == "numpy":
        rng = np.random.Generator(np.random.PCG64(seed))
        f32 = np.float32
        q = _l2n(rng.standard_normal((steps, B, H, d_k), dtype=f32))
        k = _l2n(rng.standard_normal((steps, B, H, d_k), dtype=f32))
        v = rng.standard_normal((steps, B, H, d_v), dtype=f32)
        b = _sigmoid(rng.standard_normal((steps, B, H, d_k), dtype=f32))
        w = _sigmoid(rng.standard_normal((steps, B, H, d_v), dtype=f32))
        alpha = _sigmoid(rng.standard_normal((steps, B, H, d_k), dtype=f32) + f32(alpha_mu))
        S0 = rng.standard_normal((B, H, d_k, d_v), dtype=f32) * f32(s0_std)
        out = {n: torch.from_numpy(x).to(dt).to(device)
               for n, x in dict(q=q, k=k, v=v, b=b, w=w, alpha=alpha).items()}
        out["S0"] = torch.from_numpy(S0).to(device)
        return out
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    def l2n(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    q = l2n(randn(steps, B, H, d_k)).to(dt)
    k = l2n(randn(steps, B, H, d_k)).to(dt)
    v = randn(steps, B, H, d_v).to(dt)
    b = torch.sigmoid(randn(steps, B, H, d_k)).to(dt)
    w = torch.sigmoid(randn(steps, B, H, d_v)).to(dt)
    alpha = torch.sigmoid(randn(steps, B, H, d_k) + alpha_mu).to(dt)
    S0 = randn(B, H, d_k, d_v) * s0_std
    return dict(q=q, k=k, v=v, b=b, w=w, alpha=alpha, S0=S0)


def make_inputs_torch(wl: Workload, *, device: str) -> dict:
    """As make_inputs, but drawn with a seeded torch.Generator on `device`.

    Used where host generation would dominate (the full-size benchmark workloads);
    deterministic for a given seed, with the same recipe as make_inputs.
    """
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed)
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.d_k, wl.d_v
    dt = _torch_dtype(wl.dtype)

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    def l2n(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    q = l2n(randn(B, T, H, dk)).to(dt)
    k = l2n(randn(B, T, H, dk)).to(dt)
    v = randn(B, T, H, dv).to(dt)
    b = torch.sigmoid(randn(B, T, H, dk)).to(dt)
    w = torch.sigmoid(randn(B, T, H, dv)).to(dt)
    a_shape = (B, T, H) if wl.gates == "gdn" else (B, T, H, dk)
    alpha = torch.sigmoid(randn(*a_shape) + wl.alpha_mu).to(dt)
    S0 = randn(B, H, dk, dv) * wl.s0_std if wl.s0_std > 0 else None
    beta_scalar = wl.gates in ("gdn", "kda")
    if beta_scalar:
        b = torch.sigmoid(randn(B, T, H)).to(dt)
        w = None
    return dict(q=q, k=k, v=v, alpha=alpha, b=b, w=w, S0=S0,
                alpha_scalar=(wl.gates == "gdn"), beta_scalar=beta_scalar)


def _distinct_slots(rng, rows: int, N: int, m: int) -> np.ndarray:
    """rows x m slot indices in [0, N), distinct within each row, uniformly drawn."""
    if N <= 8192:  # the first m of a random order of all N slots
        return np.argpartition(rng.random((rows, N), dtype=np.float32), m - 1, axis=1)[:, :m].astype(np.int32)
    out = rng.integers(0, N, (rows, m), dtype=np.int64)
    while True:  # redraw repeated entries until every row is distinct
        srt = np.sort(out, axis=1)
        dup_rows = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
        if dup_rows.size == 0:
            return out.astype(np.int32)
        for r in dup_rows:
            _, first = np.unique(out[r], return_index=True)
            again = np.setdiff1d(np.arange(m), first)
            out[r, again] = rng.integers(0, N, again.size)


def make_sdm_inputs(B: int, T: int, H: int, d_k: int, d_v: int, n: int, W: int, R: int, *, seed: int,
                    dtype: str = "bf16", alpha_mu: float = 3.0, m0_std: float = 0.1,
                    with_memory: bool = True, device: str = "cpu") -> dict:
    """Seeded inputs of the sparse delta memory (aiweekly.co, "Meta FAIR dévoile SDM ...": N slots
    addressed by product keys, W write and R read slots per token).

    q, k = L2normalize(N(0,1)) [B, T, H, d_k]; v = N(0,1), w = sigmoid(N(0,1)) [B, T, H, d_v];
    alpha = sigmoid(N(alpha_mu, 1)), b = sigmoid(N(0,1)) per token [B, T, H]; sub-key tables
    C1, C2 = N(0,1) [H, n, d_k/2]; M0 = N(0, m0_std^2) [B, H, N = n^2, d_v] float32 (zeros when
    m0_std = 0, None without with_memory; the draws after it do not depend on it). Independent addresses for the update alone: widx [B, T, H, W] and ridx [B, T, H, R]
    uniform distinct slots per token, weights wwt, rwt the softmax of N(0, 2^2) draws (positive,
    summing to one like the product-key weights). Draw order: q, k, v, w, alpha, b, C1, C2, M0,
    widx, wwt, ridx, rwt. Token inputs and tables are rounded to bf16 when dtype is bf16.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    N = n * n
    q = _l2n(rng.standard_normal((B, T, H, d_k), dtype=f32))
    k = _l2n(rng.standard_normal((B, T, H, d_k), dtype=f32))
    v = rng.standard_normal((B, T, H, d_v), dtype=f32)
    w = _sigmoid(rng.standard_normal((B, T, H, d_v), dtype=f32))
    alpha = _sigmoid(rng.standard_normal((B, T, H), dtype=f32) + f32(alpha_mu))
    b = _sigmoid(rng.standard_normal((B, T, H), dtype=f32))
    C1 = rng.standard_normal((H, n, d_k // 2), dtype=f32)
    C2 = rng.standard_normal((H, n, d_k // 2), dtype=f32)
    if not with_memory:  # the caller makes the memory itself (e.g. on the device, at full size)
        M0 = None
    elif m0_std > 0:
        M0 = rng.standard_normal((B, H, N, d_v), dtype=f32) * f32(m0_std)
    else:
        M0 = np.zeros((B, H, N, d_v), dtype=f32)
    rows = B * T * H

    def weights(m):
        z = rng.standard_normal((rows, m), dtype=f32) * f32(2.0)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        return (e / e.sum(axis=1, keepdims=True)).astype(f32).reshape(B, T, H, m)

    widx = _distinct_slots(rng, rows, N, W).reshape(B, T, H, W)
    wwt = weights(W)
    ridx = _distinct_slots(rng, rows, N, R).reshape(B, T, H, R)
    rwt = weights(R)
    dt = _torch_dtype(dtype)

    def t(x, to=dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(to).to(device)

    return dict(q=t(q), k=t(k), v=t(v), w=t(w), alpha=t(alpha), b=t(b), C1=t(C1), C2=t(C2),
                M0=t(M0, torch.float32), widx=t(widx, torch.int32), wwt=t(wwt, torch.float32),
                ridx=t(ridx, torch.int32), rwt=t(rwt, torch.float32), N=N)
