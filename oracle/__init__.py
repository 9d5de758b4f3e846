"""fp64 CPU oracle for the Gated DeltaNet-2 recurrence.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package. The product path (``gated_delta_rule_25_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``gdn2_oracle.c`` (plain C, float64, one token at a time); this
module only compiles it with gcc, converts arrays to contiguous float64 and calls it.

Source of the update rule: the page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами
для раздельного стирания и записи в линейном внимании", paragraph "Техническая схема",
state-update equation S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T.
The readout o_t = S_t^T q_t (updated state) is a reading, not printed on the pages.

``backward`` (reverse mode of the same recurrence) is pinned by ``tests/oracle_bwd_pins.py``
against finite differences, a closed form, the affine dependence on S0 and automatic
differentiation of a transition-matrix formulation.
``pkm_address`` / ``sdm_forward`` / ``sdm_step`` (the sparse delta memory, numpy float64, in
``sdm.py`` with its readings) are pinned by ``tests/test_oracle_sdm.py``.
``rmsnorm`` / ``rmsnorm_backward`` (the output normalisation, numpy float64) are pinned by
``tests/test_oracle_rmsnorm.py`` against closed forms, invariants and finite differences.
Every forward function is pinned by ``tests/test_oracle_pins.py`` against a hand-worked example,
brute-force transition products, closed forms and textbook special cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn2_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False, out_path: str | None = None, src_path: str | None = None) -> str:
    """Compile the C oracle with gcc (plain -O2, IEEE arithmetic, no -ffast-math)."""
    out = out_path or _LIB_PATH
    src = src_path or _SRC
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", tmp, src, "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def load_library(path: str | None = None):
    """Load (building first if needed) the oracle library; returns a ctypes handle."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
        _declare(lib)
        return lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            _declare(lib)
            _lib = lib
    return _lib


def _declare(lib) -> None:
    p = ctypes.c_void_p
    L = ctypes.c_long
    lib.gdn2_oracle_forward.argtypes = [p, p, p, p, p, p, p, p, p, L, L, L, L, L, ctypes.c_int]
    lib.gdn2_oracle_forward.restype = ctypes.c_int
    lib.gdn2_oracle_backward.argtypes = [p] * 16 + [L, L, L, L, L, ctypes.c_int]
    lib.gdn2_oracle_backward.restype = ctypes.c_int


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: exact upcast on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, alpha, b, w, S0=None, *, threads: int | None = None, lib=None):
    """Run the recurrence over [B, T, H, d] inputs in float64.

    q, k, alpha, b: [B, T, H, d_k]; v, w: [B, T, H, d_v]; S0: [B, H, d_k, d_v] or None (zeros).
    Scalar-gate forms (Gated DeltaNet / KDA) are passed here already broadcast to these
    shapes (see ``broadcast_gates``). Returns (o [B, T, H, d_v], S_T [B, H, d_k, d_v]) as
    float64 numpy arrays. Inputs may be numpy arrays or CPU/GPU torch tensors; values are
    upcast exactly to float64.
    """
    q, k, v, alpha, b, w = (_f64(x) for x in (q, k, v, alpha, b, w))
    S0 = _f64(S0)
    if q.ndim != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, x, d in (("k", k, dk), ("alpha", alpha, dk), ("b", b, dk), ("v", v, dv), ("w", w, dv)):
        if x.shape != (B, T, H, d):
            raise ValueError(f"{name} has shape {x.shape}, expected {(B, T, H, d)}")
    if S0 is not None and S0.shape != (B, H, dk, dv):
        raise ValueError(f"S0 has shape {S0.shape}, expected {(B, H, dk, dv)}")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_T = np.zeros((B, H, dk, dv), dtype=np.float64)
    lib = lib or load_library()
    rc = lib.gdn2_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                 _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv,
                                 int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn2_oracle_forward failed with status {rc}")
    return o, S_T


def decode_step(q, k, v, alpha, b, w, S, *, threads: int | None = None, lib=None):
    """One single-token step: inputs [B, H, d], state S [B, H, d_k, d_v].

    This is ``forward`` with T = 1. Returns (o [B, H, d_v], S_new [B, H, d_k, d_v]).
    """
    xs = [_f64(x) for x in (q, k, v, alpha, b, w)]
    xs = [x[:, None] for x in xs]  # [B, H, d] -> [B, 1, H, d]
    o, S_new = forward(*xs, S0=S, threads=threads, lib=lib)
    return o[:, 0], S_new


def broadcast_gates(alpha, b, w, d_k: int, d_v: int, *, alpha_scalar: bool, beta_scalar: bool):
    """Materialise scalar gates as the per-channel gates the general rule takes.

    Gated DeltaNet and KDA are the general rule with collapsed gates: with one scalar
    beta_t, b_t = beta_t * 1_{d_k} and w_t = beta_t * 1_{d_v}; Gated DeltaNet also has a
    scalar decay alpha_t broadcast over the key channels (page "NVIDIA улучшила память LLM
    без роста затрат на контекст", the authors' quote on the earlier models as special
    cases). alpha / b given as [..., 1] or [...] scalars per (b, t, h); w is ignored when
    beta_scalar is set.
    """
    alpha = _f64(alpha)
    b = _f64(b)
    if alpha_scalar:
        a = alpha if alpha.shape[-1:] == (1,) else alpha[..., None]
        alpha = np.broadcast_to(a, a.shape[:-1] + (d_k,)).copy()
    if beta_scalar:
        be = b if b.shape[-1:] == (1,) else b[..., None]
        b = np.broadcast_to(be, be.shape[:-1] + (d_k,)).copy()
        w = np.broadcast_to(be, be.shape[:-1] + (d_v,)).copy()
    else:
        w = _f64(w)
    return alpha, b, w


def backward(q, k, v, alpha, b, w, S0=None, dO=None, dS_T=None, *, threads: int | None = None, lib=None):
    """Gradients of L = sum_t <dO_t, o_t> + <dS_T, S_T> in float64 (reverse mode of the
    recurrence, token by token; see gdn2_oracle.c).

    Shapes as in ``forward``; dO: [B, T, H, d_v] or None (zeros); dS_T: [B, H, d_k, d_v] or None.
    Returns a dict with dq, dk, dalpha, db ([B, T, H, d_k]), dv, dw ([B, T, H, d_v]) and dS0
    ([B, H, d_k, d_v]) as float64 numpy arrays.
    """
    q, k, v, alpha, b, w = (_f64(x) for x in (q, k, v, alpha, b, w))
    S0, dO, dS_T = _f64(S0), _f64(dO), _f64(dS_T)
    if q.ndim != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, x, d in (("k", k, dk), ("alpha", alpha, dk), ("b", b, dk), ("v", v, dv), ("w", w, dv)):
        if x.shape != (B, T, H, d):
            raise ValueError(f"{name} has shape {x.shape}, expected {(B, T, H, d)}")
    if dO is not None and dO.shape != (B, T, H, dv):
        raise ValueError(f"dO has shape {dO.shape}, expected {(B, T, H, dv)}")
    for name, x in (("S0", S0), ("dS_T", dS_T)):
        if x is not None and x.shape != (B, H, dk, dv):
            raise ValueError(f"{name} has shape {x.shape}, expected {(B, H, dk, dv)}")
    out = {n: np.zeros((B, T, H, dk)) for n in ("dq", "dk", "dalpha", "db")}
    out.update({n: np.zeros((B, T, H, dv)) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((B, H, dk, dv))
    lib = lib or load_library()
    rc = lib.gdn2_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                                  _ptr(dO), _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]),
                                  _ptr(out["dalpha"]), _ptr(out["db"]), _ptr(out["dv"]),
                                  _ptr(out["dw"]), _ptr(out["dS0"]), B, T, H, dk, dv,
                                  int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn2_oracle_backward failed with status {rc}")
    return out


def prologue(q, k, alpha, b, w, *, l2norm: bool, gate_logits: bool):
    """The steps in front of the recurrence, in float64: q and k L2-normalised per token and head
    over d_k (x / max(||x||, 1e-12)), and the gates taken through the logistic sigmoid from their
    pre-activations (page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …",
    paragraph "Архитектурно": L2-normalised q/k and sigmoid gates). w may be None (scalar beta
    carried in b). Returns (q, k, alpha, b, w) as float64 numpy arrays.
    """
    q, k, alpha, b = (_f64(x) for x in (q, k, alpha, b))
    w = _f64(w)
    if l2norm:
        q = q / np.maximum(np.sqrt(np.sum(q * q, axis=-1, keepdims=True)), 1e-12)
        k = k / np.maximum(np.sqrt(np.sum(k * k, axis=-1, keepdims=True)), 1e-12)
    if gate_logits:
        sig = lambda x: 1.0 / (1.0 + np.exp(-x))
        alpha, b = sig(alpha), sig(b)
        w = None if w is None else sig(w)
    return q, k, alpha, b, w


def prologue_backward(q, k, alpha, b, w, grads: dict, *, l2norm: bool, gate_logits: bool) -> dict:
    """Gradients with respect to the raw inputs of prologue(), given the gradients `grads` (dq,
    dk, dalpha, db and, when w is given, dw) with respect to its outputs; float64 (parity
    pinned by finite differences of prologue() itself). For x_n = x / max(|x|, 1e-12):
    dx = (dx_n - (dx_n . x_n) x_n) / |x| when |x| > 1e-12, else dx_n / 1e-12. For a = sigma(x):
    dx = da * a (1 - a). Returns a dict with the same keys.
    """
    q, k, alpha, b = (_f64(x) for x in (q, k, alpha, b))
    w = _f64(w)
    out = {n: _f64(v) for n, v in grads.items()}
    if l2norm:
        for name, x in (("dq", q), ("dk", k)):
            nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            big = nrm > 1e-12
            xn = x / np.maximum(nrm, 1e-12)
            g = out[name]
            proj = g - np.sum(g * xn, axis=-1, keepdims=True) * xn
            out[name] = np.where(big, proj / np.maximum(nrm, 1e-12), g / 1e-12)
    if gate_logits:
        sig = lambda x: 1.0 / (1.0 + np.exp(-x))
        for name, x in (("dalpha", alpha), ("db", b), ("dw", w)):
            if x is not None and name in out:
                s = sig(x)
                out[name] = out[name] * s * (1.0 - s)
    return out


def rmsnorm(x, weight=None, *, eps: float):
    """The RMS normalisation the recurrent layer's output passes through (page "NVIDIA
    представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph "Архитектурно"), per row
    over the last axis (one head's d_v outputs of one token), in float64:
    y = x / sqrt(mean(x^2) + eps) * weight; weight None means ones.
    """
    x = _f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return y if weight is None else y * _f64(weight)


def rmsnorm_backward(x, weight, dy, *, eps: float) -> dict:
    """Gradients of L = sum(dy * rmsnorm(x, weight)) with respect to x and weight, float64 (pinned
    by central differences of rmsnorm() itself). With r = (mean(x^2) + eps)^(-1/2),
    xh = x r and u = dy * weight: dx = r (u - xh mean(xh u)) per row, and dweight = the sum of
    dy * xh over every row.
    """
    x, dy = _f64(x), _f64(dy)
    g = np.ones(x.shape[-1]) if weight is None else _f64(weight)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = x * r
    u = dy * g
    dx = r * (u - xh * np.mean(xh * u, axis=-1, keepdims=True))
    dweight = (dy * xh).reshape(-1, x.shape[-1]).sum(axis=0)
    return dict(dx=dx, dweight=dweight)


from .sdm import pkm_address, sdm_forward, sdm_step  # noqa: E402  (the sparse delta memory, numpy float64)
