"""Gated DeltaNet-2 recurrence on AMD Instinct MI355X: thin Python binding of libgdn2.so.

The compute lives in the C-ABI library (include/gdn2.h, HIP kernels for gfx950). This module
only checks tensor metadata, passes device pointers and the current HIP stream, and turns
status codes into exceptions. PyTorch provides device memory and streams. There is no fallback:
if the library is not built or no GPU is present, calls raise.

    o, S_T = chunk_fwd(q, k, v, alpha, b, w, S0)        # prefill, chunk length 64
    o, S_T = recurrent_fwd(q, k, v, alpha, b, w, S0)    # token-by-token fp32 prefill
    o = decode_step(q, k, v, alpha, b, w, S)            # one token, S updated in place
    g = chunk_bwd(q, k, v, alpha, b, w, S0, dO, dS_T)    # gradients (dict: dq, dk, dv, ...)
    o, S_T = chunk_fwd_varlen(q, k, v, alpha, b, w, cu_seqlens, S0)  # packed [T_total, H, d] rows
    g = chunk_bwd_varlen(q, k, v, alpha, b, w, cu_seqlens, S0, dO, dS_T)
    y = rmsnorm_fwd(o, weight, eps=1e-6)                # output RMS norm per head row

Shapes: q, k, alpha, b [B, T, H, d_k]; v, w [B, T, H, d_v]; states [B, H, d_k, d_v] float32;
decode drops the T axis. Scalar gates: alpha [B, T, H] (alpha_scalar) and b = beta [B, T, H]
with w None (beta_scalar) -- inferred from the shapes.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime before libgdn2.so binds to it)

__all__ = ["chunk_fwd", "chunk_fwd_varlen", "chunk_fwd_varlen_workspace_bytes", "recurrent_fwd", "decode_step", "chunk_fwd_workspace_bytes", "chunk_bwd",
           "chunk_bwd_workspace_bytes", "chunk_bwd_varlen", "chunk_bwd_varlen_workspace_bytes",
           "Gdn2Error", "library_path", "load", "ALPHA_SCALAR", "BETA_SCALAR", "QK_L2NORM", "GATE_LOGITS",
           "decode_step_slots", "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_noalloc",
           "sdm_address", "sdm_state", "sdm_fwd", "sdm_fold", "chunk_fwd_save", "chunk_fwd_varlen_save"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn2.so")
_lib = None

BF16, F32 = 0, 1
ALPHA_SCALAR, BETA_SCALAR, QK_L2NORM, GATE_LOGITS = 1, 2, 4, 8
_STATUS = {0: "GDN2_OK", 1: "GDN2_ERR_NULL", 2: "GDN2_ERR_SHAPE", 3: "GDN2_ERR_UNSUPPORTED",
           4: "GDN2_ERR_ALIGN", 5: "GDN2_ERR_ALIAS", 6: "GDN2_ERR_HIP", 7: "GDN2_ERR_WORKSPACE",
           8: "GDN2_ERR_SCRATCH"}


class Gdn2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdn2.so (built by gated_delta_rule_25_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m gated_delta_rule_25_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    lib.gdn2_chunk_fwd.argtypes = [p] * 9 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_fwd.restype = ctypes.c_int
    lib.gdn2_chunk_fwd_workspace_bytes.argtypes = [i32] * 5 + [ctypes.c_int, u32]
    lib.gdn2_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn2_chunk_fwd_varlen.argtypes = [p] * 10 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_fwd_varlen.restype = ctypes.c_int
    lib.gdn2_chunk_fwd_varlen_workspace_bytes.argtypes = [i32] * 5 + [ctypes.c_int, u32]
    lib.gdn2_chunk_fwd_varlen_workspace_bytes.restype = sz
    lib.gdn2_chunk_bwd.argtypes = [p] * 16 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_bwd.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_workspace_bytes.argtypes = [i32] * 5 + [ctypes.c_int, u32]
    lib.gdn2_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn2_chunk_fwd_save.argtypes = [p] * 9 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_fwd_save.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_saved.argtypes = [p] * 16 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_bwd_saved.restype = ctypes.c_int
    lib.gdn2_chunk_fwd_varlen_save.argtypes = [p] * 10 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_fwd_varlen_save.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_varlen_saved.argtypes = [p] * 17 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_bwd_varlen_saved.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_varlen.argtypes = [p] * 17 + [i32] * 5 + [ctypes.c_int, u32, p, sz, p]
    lib.gdn2_chunk_bwd_varlen.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_varlen_workspace_bytes.argtypes = [i32] * 5 + [ctypes.c_int, u32]
    lib.gdn2_chunk_bwd_varlen_workspace_bytes.restype = sz
    lib.gdn2_decode_step_slots.argtypes = [p] * 9 + [i32] * 5 + [ctypes.c_int, u32, p]
    lib.gdn2_decode_step_slots.restype = ctypes.c_int
    lib.gdn2_recurrent_fwd.argtypes = [p] * 9 + [i32] * 5 + [ctypes.c_int, u32, p]
    lib.gdn2_recurrent_fwd.restype = ctypes.c_int
    lib.gdn2_decode_step.argtypes = [p] * 8 + [i32] * 4 + [ctypes.c_int, u32, p]
    lib.gdn2_decode_step.restype = ctypes.c_int
    i64, f32 = ctypes.c_int64, ctypes.c_float
    lib.gdn2_rmsnorm_fwd.argtypes = [p] * 3 + [i64, i32, f32, ctypes.c_int, p]
    lib.gdn2_rmsnorm_fwd.restype = ctypes.c_int
    lib.gdn2_rmsnorm_bwd.argtypes = [p] * 5 + [i64, i32, f32, p, sz, p]
    lib.gdn2_rmsnorm_bwd.restype = ctypes.c_int
    lib.gdn2_rmsnorm_bwd_noalloc.argtypes = [p] * 5 + [i64, i32, f32, p]
    lib.gdn2_rmsnorm_bwd_noalloc.restype = ctypes.c_int
    lib.gdn2_rmsnorm_bwd_workspace_bytes.argtypes = [i64, i32]
    lib.gdn2_rmsnorm_bwd_workspace_bytes.restype = sz
    lib.gdn2_sdm_address.argtypes = [p, p, p, i64, i32, i32, i32, i32, i32, p, p, p]
    lib.gdn2_sdm_address.restype = ctypes.c_int
    lib.gdn2_sdm_fwd.argtypes = [p] * 12 + [i32, i32, i32, i64, i32, i32, i32, i32, p]
    lib.gdn2_sdm_fwd.restype = ctypes.c_int
    lib.gdn2_sdm_fold.argtypes = [p, p, p, i32, i32, i64, i32, p]
    lib.gdn2_sdm_fold.restype = ctypes.c_int
    lib.gdn2_status_str.argtypes = [ctypes.c_int]
    lib.gdn2_status_str.restype = ctypes.c_char_p
    lib.gdn2_abi_version.argtypes = []
    lib.gdn2_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported input dtype {t.dtype} (bfloat16 or float32)")


def _prologue_flags(l2norm: bool, gate_logits: bool) -> int:
    return (QK_L2NORM if l2norm else 0) | (GATE_LOGITS if gate_logits else 0)


def _check_inputs(q, k, v, alpha, b, w, ndim_tok: int):
    ins = [x for x in (q, k, v, alpha, b, w) if x is not None]
    dt = q.dtype
    for x in ins:
        if not x.is_cuda:
            raise ValueError("inputs must be GPU tensors")
        if not x.is_contiguous():
            raise ValueError("inputs must be contiguous")
        if x.dtype != dt:
            raise TypeError("q, k, v, alpha, b, w must share one dtype")
    if q.dim() != ndim_tok:
        raise ValueError(f"q must have {ndim_tok} dimensions")
    flags = 0
    if alpha.dim() == ndim_tok - 1:
        flags |= ALPHA_SCALAR
    if w is None:
        if b.dim() != ndim_tok - 1:
            raise ValueError("w may be None only with a scalar beta passed as b")
        flags |= BETA_SCALAR
    return flags


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _scratch(nbytes, device, stream):
    """A temporary workspace allocated on the stream the kernels run on, so that once it is
    freed here the caching allocator hands it out again only in that stream's order."""
    if stream is None:
        return torch.empty(nbytes, device=device, dtype=torch.uint8)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, device=device, dtype=torch.uint8)


def _state_out(S0, B, H, dk, dv, device, S_out):
    if S_out is None:
        S_out = torch.empty(B, H, dk, dv, device=device, dtype=torch.float32)
    if S0 is not None and (S0.dtype != torch.float32 or not S0.is_contiguous()):
        raise TypeError("S0 must be a contiguous float32 tensor")
    return S_out


def chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, dtype=torch.bfloat16, flags=0) -> int:
    """Workspace bytes of gdn2_chunk_fwd's two-kernel path at these sizes (0: it does not take them)."""
    return int(load().gdn2_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v,
                                                     BF16 if dtype == torch.bfloat16 else F32,
                                                     flags))


def chunk_fwd(q, k, v, alpha, b, w=None, S0=None, *, o=None, S_out=None, workspace=None,
              schedule="split", l2norm=False, gate_logits=False, stream=None):
    """Chunkwise prefill (C = 64). Returns (o [B, T, H, d_v] fp32, S_T [B, H, d_k, d_v]).

    schedule: "split" (the default) passes the two-kernel path's workspace where it takes the sizes
    (allocated here unless given); "fused" passes none: the fused kernel, allocating nothing (or the
    single kernel for sizes the fused kernel does not take). l2norm / gate_logits: the kernels
    normalise q, k and take the gates through the sigmoid themselves.
    """
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 4) | _prologue_flags(l2norm, gate_logits)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty(B, T, H, dv, device=q.device, dtype=torch.float32)
    S_out = _state_out(S0, B, H, dk, dv, q.device, S_out)
    dt = _dtype_code(q)
    if schedule not in ("fused", "split"):
        raise ValueError("schedule must be 'split' or 'fused'")
    need = 0 if schedule == "fused" else int(lib.gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, dt, flags))
    if need and workspace is None:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                            _ptr(o), _ptr(S_out), B, T, H, dk, dv, dt, flags, _ptr(workspace),
                            ws_bytes, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_fwd", st)
    return o, S_out


def chunk_fwd_save(q, k, v, alpha, b, w=None, S0=None, *, o=None, S_out=None, workspace=None,
                   l2norm=False, gate_logits=False, stream=None):
    """The forward of a training step (gdn2_chunk_fwd_save): (o, S_T) as chunk_fwd computes them,
    and the backward workspace, which then holds what chunk_bwd(..., saved=workspace) reads
    instead of recomputing the forward. Returns (o, S_T, workspace); the workspace is allocated
    here unless given (gdn2_chunk_bwd_workspace_bytes for these sizes and flags)."""
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 4) | _prologue_flags(l2norm, gate_logits)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty(B, T, H, dv, device=q.device, dtype=torch.float32)
    S_out = _state_out(S0, B, H, dk, dv, q.device, S_out)
    dt = _dtype_code(q)
    need = int(lib.gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, dt, flags))
    if need and workspace is None:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn2_chunk_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                                 _ptr(o), _ptr(S_out), B, T, H, dk, dv, dt, flags, _ptr(workspace),
                                 ws_bytes, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_fwd_save", st)
    return o, S_out, workspace


def chunk_fwd_varlen_workspace_bytes(N, T_total, H, d_k, d_v, dtype=torch.bfloat16, flags=0) -> int:
    return int(load().gdn2_chunk_fwd_varlen_workspace_bytes(N, T_total, H, d_k, d_v,
                                                            BF16 if dtype == torch.bfloat16 else F32,
                                                            flags))


def chunk_fwd_varlen(q, k, v, alpha, b, w, cu_seqlens, S0=None, *, o=None, S_out=None, workspace=None,
                     l2norm=False, gate_logits=False, stream=None):
    """Prefill of N = len(cu_seqlens) - 1 sequences packed along the token axis.

    q, k, alpha, b [T_total, H, d_k]; v, w [T_total, H, d_v] (scalar gates [T_total, H]);
    cu_seqlens int32 on the GPU, sequence s = rows cu_seqlens[s] .. cu_seqlens[s+1] - 1;
    S0 [N, H, d_k, d_v] or None. Returns (o [T_total, H, d_v] fp32, S_T [N, H, d_k, d_v]).
    """
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 3) | _prologue_flags(l2norm, gate_logits)
    T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or not cu_seqlens.is_cuda \
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise TypeError("cu_seqlens must be a contiguous 1-d int32 GPU tensor of N + 1 entries")
    N = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty(T, H, dv, device=q.device, dtype=torch.float32)
    S_out = _state_out(S0, N, H, dk, dv, q.device, S_out)
    dt = _dtype_code(q)
    if workspace is None:
        need = int(lib.gdn2_chunk_fwd_varlen_workspace_bytes(N, T, H, dk, dv, dt, flags))
        if need == 0:
            raise Gdn2Error("gdn2_chunk_fwd_varlen", 3)
        workspace = _scratch(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.gdn2_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                                   _ptr(o), _ptr(S_out), _ptr(cu_seqlens), N, T, H, dk, dv, dt, flags,
                                   _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_fwd_varlen", st)
    return o, S_out


def chunk_fwd_varlen_save(q, k, v, alpha, b, w, cu_seqlens, S0=None, *, o=None, S_out=None, workspace=None,
                          l2norm=False, gate_logits=False, stream=None):
    """The packed forward of a training step (gdn2_chunk_fwd_varlen_save): (o, S_T) as
    chunk_fwd_varlen computes them, and the backward workspace holding what
    chunk_bwd_varlen(..., saved=workspace) reads. Returns (o, S_T, workspace)."""
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 3) | _prologue_flags(l2norm, gate_logits)
    T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or not cu_seqlens.is_cuda \
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise TypeError("cu_seqlens must be a contiguous 1-d int32 GPU tensor of N + 1 entries")
    N = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty(T, H, dv, device=q.device, dtype=torch.float32)
    S_out = _state_out(S0, N, H, dk, dv, q.device, S_out)
    dt = _dtype_code(q)
    need = int(lib.gdn2_chunk_bwd_varlen_workspace_bytes(N, T, H, dk, dv, dt, flags))
    if need and workspace is None:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn2_chunk_fwd_varlen_save(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                                        _ptr(o), _ptr(S_out), _ptr(cu_seqlens), N, T, H, dk, dv, dt, flags,
                                        _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_fwd_varlen_save", st)
    return o, S_out, workspace


def chunk_bwd_workspace_bytes(B, T, H, d_k, d_v, dtype=torch.bfloat16, flags=0) -> int:
    return int(load().gdn2_chunk_bwd_workspace_bytes(B, T, H, d_k, d_v,
                                                     BF16 if dtype == torch.bfloat16 else F32, flags))


def chunk_bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None, *, workspace=None, out=None, l2norm=False,
              gate_logits=False, saved=None, stream=None):
    """Gradients of sum <dO, o> + <dS_T, S_T> for the prefill (bf16 inputs).

    Returns a dict of float32 tensors: dq, dk, dalpha, db [B, T, H, d_k], dv, dw [B, T, H, d_v] and
    dS0 [B, H, d_k, d_v]. Scalar gates (alpha [B, T, H]; beta passed as b [B, T, H] with w None)
    give dalpha [B, T, H], and db [B, T, H] = dL/dbeta with no dw. With l2norm / gate_logits the
    inputs are the raw ones the forward takes with the same flags, and the gradients are with
    respect to them. `out` may supply any of them; the workspace is allocated here unless given.
    saved: the workspace a chunk_fwd_save call on the same inputs returned (gdn2_chunk_bwd_saved):
    the forward is then read from it, not recomputed.
    """
    if saved is not None:
        if workspace is not None and workspace is not saved:
            raise ValueError("pass the saved workspace as `saved` alone")
        return _bwd(q, k, v, alpha, b, w, S0, dO, dS_T, None, saved, out, l2norm, gate_logits, stream,
                    fn="gdn2_chunk_bwd_saved")
    return _bwd(q, k, v, alpha, b, w, S0, dO, dS_T, None, workspace, out, l2norm, gate_logits, stream)


def chunk_bwd_varlen_workspace_bytes(N, T_total, H, d_k, d_v, dtype=torch.bfloat16, flags=0) -> int:
    return int(load().gdn2_chunk_bwd_varlen_workspace_bytes(N, T_total, H, d_k, d_v,
                                                            BF16 if dtype == torch.bfloat16 else F32, flags))


def chunk_bwd_varlen(q, k, v, alpha, b, w, cu_seqlens, S0, dO, dS_T=None, *, workspace=None, out=None,
                     l2norm=False, gate_logits=False, saved=None, stream=None):
    """Gradients for the packed prefill chunk_fwd_varlen: the rows are [T_total, H, d] and the
    states [N, H, d_k, d_v], N = len(cu_seqlens) - 1; otherwise as chunk_bwd (saved: the workspace
    a chunk_fwd_varlen_save call on the same inputs returned)."""
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or not cu_seqlens.is_cuda \
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise TypeError("cu_seqlens must be a contiguous 1-d int32 GPU tensor of N + 1 entries")
    if saved is not None:
        if workspace is not None and workspace is not saved:
            raise ValueError("pass the saved workspace as `saved` alone")
        return _bwd(q, k, v, alpha, b, w, S0, dO, dS_T, cu_seqlens, saved, out, l2norm, gate_logits, stream,
                    fn="gdn2_chunk_bwd_varlen_saved")
    return _bwd(q, k, v, alpha, b, w, S0, dO, dS_T, cu_seqlens, workspace, out, l2norm, gate_logits, stream)


def _bwd(q, k, v, alpha, b, w, S0, dO, dS_T, cu, workspace, out, l2norm, gate_logits, stream, fn=None):
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 4 if cu is None else 3) | _prologue_flags(l2norm, gate_logits)
    lead = tuple(q.shape[:-2])  # (B, T), or (T_total,) for a packed batch
    H, dk = q.shape[-2:]
    dv = v.shape[-1]
    B, T = lead if cu is None else (cu.numel() - 1, lead[0])  # sequences (states), rows per call
    for name, x in (("S0", S0), ("dO", dO), ("dS_T", dS_T)):
        if x is not None and (x.dtype != torch.float32 or not x.is_contiguous() or not x.is_cuda):
            raise TypeError(f"{name} must be a contiguous float32 GPU tensor")
    out = dict(out or {})
    f32 = dict(device=q.device, dtype=torch.float32)
    for name in ("dq", "dk"):
        out.setdefault(name, torch.empty(*lead, H, dk, **f32))
    out.setdefault("dalpha", torch.empty(*lead, H, **f32) if flags & ALPHA_SCALAR else torch.empty(*lead, H, dk, **f32))
    out.setdefault("db", torch.empty(*lead, H, **f32) if flags & BETA_SCALAR else torch.empty(*lead, H, dk, **f32))
    out.setdefault("dv", torch.empty(*lead, H, dv, **f32))
    if not flags & BETA_SCALAR:
        out.setdefault("dw", torch.empty(*lead, H, dv, **f32))
    out.setdefault("dS0", torch.empty(B, H, dk, dv, **f32))
    dt = _dtype_code(q)
    base = "gdn2_chunk_bwd" if cu is None else "gdn2_chunk_bwd_varlen"
    fn = fn or base
    need = int(getattr(lib, base + "_workspace_bytes")(B, T, H, dk, dv, dt, flags))
    if need and workspace is None:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(dO), _ptr(dS_T),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["db"]),
            _ptr(out.get("dw")), _ptr(out["dS0"])]
    if cu is not None:
        args.append(_ptr(cu))
    st = getattr(lib, fn)(*args, B, T, H, dk, dv, dt, flags, _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise Gdn2Error(fn, st)
    return out


def recurrent_fwd(q, k, v, alpha, b, w=None, S0=None, *, o=None, S_out=None, l2norm=False,
                  gate_logits=False, stream=None):
    """Token-by-token fp32 prefill. Returns (o, S_T) like chunk_fwd."""
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 4) | _prologue_flags(l2norm, gate_logits)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty(B, T, H, dv, device=q.device, dtype=torch.float32)
    S_out = _state_out(S0, B, H, dk, dv, q.device, S_out)
    st = lib.gdn2_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                _ptr(S0), _ptr(o), _ptr(S_out), B, T, H, dk, dv, _dtype_code(q),
                                flags, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_recurrent_fwd", st)
    return o, S_out


def decode_step(q, k, v, alpha, b, w, S, *, o=None, l2norm=False, gate_logits=False, stream=None):
    """One decode step on [B, H, d] inputs; updates S [B, H, d_k, d_v] in place, returns o."""
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 3) | _prologue_flags(l2norm, gate_logits)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if S.dtype != torch.float32 or not S.is_contiguous():
        raise TypeError("S must be a contiguous float32 tensor")
    if o is None:
        o = torch.empty(B, H, dv, device=q.device, dtype=torch.float32)
    st = lib.gdn2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S),
                              _ptr(o), B, H, dk, dv, _dtype_code(q), flags, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_decode_step", st)
    return o


def decode_step_slots(q, k, v, alpha, b, w, S_pool, slots, *, o=None, l2norm=False, gate_logits=False,
                      stream=None):
    """One decode step over a state pool: batch row i updates S_pool[slots[i]] in place
    (S_pool [n_slots, H, d_k, d_v] float32, slots [B] int32 on the GPU; rows whose slot is outside
    the pool are skipped). Returns o [B, H, d_v]."""
    lib = load()
    flags = _check_inputs(q, k, v, alpha, b, w, 3) | _prologue_flags(l2norm, gate_logits)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if S_pool.dtype != torch.float32 or not S_pool.is_contiguous():
        raise TypeError("S_pool must be a contiguous float32 tensor")
    if slots.dtype != torch.int32 or not slots.is_contiguous() or not slots.is_cuda or slots.numel() != B:
        raise TypeError("slots must be a contiguous int32 GPU tensor of B entries")
    if o is None:
        o = torch.empty(B, H, dv, device=q.device, dtype=torch.float32)
    st = lib.gdn2_decode_step_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S_pool),
                                    _ptr(slots), _ptr(o), B, H, dk, dv, S_pool.shape[0], _dtype_code(q),
                                    flags, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_decode_step_slots", st)
    return o


def _norm_rows(x, name):
    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 GPU tensor")
    d = x.shape[-1]
    return x.numel() // d if d else 0, d


def rmsnorm_fwd(x, weight=None, *, eps: float = 1e-6, out=None, out_dtype=torch.float32, stream=None):
    """Output RMS norm over the last axis of x (float32, e.g. o [B, T, H, d_v]):
    y = x / sqrt(mean(x^2) + eps) * weight. out may be x itself (float32, in place)."""
    lib = load()
    rows, d = _norm_rows(x, "x")
    if weight is not None:
        _norm_rows(weight, "weight")
    if out is None:
        out = torch.empty(x.shape, device=x.device, dtype=out_dtype)
    dt = BF16 if out.dtype == torch.bfloat16 else F32
    st = lib.gdn2_rmsnorm_fwd(_ptr(x), _ptr(weight), _ptr(out), rows, d, float(eps), dt, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_rmsnorm_fwd", st)
    return out


def rmsnorm_bwd(x, weight, dy, *, eps: float = 1e-6, dx=None, need_dweight: bool = True, stream=None):
    """Gradients of rmsnorm_fwd: returns dict(dx, dweight) (dweight None unless need_dweight)."""
    lib = load()
    rows, d = _norm_rows(x, "x")
    _norm_rows(dy, "dy")
    if dx is None:
        dx = torch.empty_like(x)
    dweight = torch.empty(d, device=x.device, dtype=torch.float32) if need_dweight else None
    need = int(lib.gdn2_rmsnorm_bwd_workspace_bytes(rows, d)) if need_dweight else 0
    ws = _scratch(need, x.device, stream) if need else None
    st = lib.gdn2_rmsnorm_bwd(_ptr(x), _ptr(weight), _ptr(dy), _ptr(dx), _ptr(dweight), rows, d, float(eps),
                              _ptr(ws), need, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_rmsnorm_bwd", st)
    return dict(dx=dx, dweight=dweight)


def rmsnorm_bwd_noalloc(x, weight, dy, *, eps: float = 1e-6, dx, dweight=None, stream=None):
    """rmsnorm_bwd through gdn2_rmsnorm_bwd_noalloc: the caller passes every output (dx [rows, d],
    dweight [d] float32 or None) and the library uses its own fixed device scratch, so this call
    allocates nothing. Returns dict(dx, dweight)."""
    lib = load()
    rows, d = _norm_rows(x, "x")
    _norm_rows(dy, "dy")
    if dx is None or dx.shape != x.shape or dx.dtype != torch.float32 or not dx.is_contiguous():
        raise ValueError("dx must be a contiguous float32 tensor shaped like x")
    if dweight is not None and (dweight.dtype != torch.float32 or dweight.numel() != d or not dweight.is_contiguous()):
        raise ValueError("dweight must be a contiguous float32 tensor of d elements")
    st = lib.gdn2_rmsnorm_bwd_noalloc(_ptr(x), _ptr(weight), _ptr(dy), _ptr(dx), _ptr(dweight), rows, d, float(eps),
                                      _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_rmsnorm_bwd_noalloc", st)
    return dict(dx=dx, dweight=dweight)


def _contig(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def sdm_address(x, C1, C2, m: int, *, idx=None, weight=None, stream=None):
    """Product-key addressing (gdn2_sdm_address) of queries x [..., H, d_k] against sub-key
    tables C1, C2 [H, n, d_k/2]: returns (idx [..., H, m] int32, weight [..., H, m] float32)."""
    lib = load()
    _contig(x, "x")
    H, dk = x.shape[-2], x.shape[-1]
    rows = x.numel() // (H * dk) if x.numel() else 0
    _contig(C1, "C1", x.dtype)
    _contig(C2, "C2", x.dtype, C1.shape)
    if C1.dim() != 3 or C1.shape[0] != H or C1.shape[2] * 2 != dk:
        raise ValueError("C1, C2 must be [H, n, d_k/2]")
    n = C1.shape[1]
    shp = tuple(x.shape[:-1]) + (m,)
    if idx is None:
        idx = torch.empty(shp, device=x.device, dtype=torch.int32)
    if weight is None:
        weight = torch.empty(shp, device=x.device, dtype=torch.float32)
    st = lib.gdn2_sdm_address(_ptr(x), _ptr(C1), _ptr(C2), rows, H, dk, n, m, _dtype_code(x), _ptr(idx),
                              _ptr(weight), _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_sdm_address", st)
    return idx, weight


def sdm_state(M0):
    """The memory state gdn2_sdm_fwd takes, from an initial memory M0 [B, H, N, d_v] float32 (used
    in place): (M0, stamp [B, H, d_v/64, N] float64 zeros, L [B, H, d_v/64] float64 zeros)."""
    _contig(M0, "M0", torch.float32)
    B, H, N, dv = M0.shape
    stamp = torch.zeros(B, H, dv // 64, N, device=M0.device, dtype=torch.float64)
    L = torch.zeros(B, H, dv // 64, device=M0.device, dtype=torch.float64)
    return M0, stamp, L


def sdm_fwd(v, alpha, b, w, widx, wwt, ridx, rwt, state, *, o=None, stream=None):
    """The sparse delta memory over [B, T, H, ...] tokens (gdn2_sdm_fwd): v, w [B, T, H, d_v]
    (w None: ones), alpha, b [B, T, H]; widx/wwt [B, T, H, W], ridx/rwt [B, T, H, R]; state =
    (M, stamp, L) as sdm_state makes it, updated in place. Returns o [B, T, H, d_v] float32."""
    lib = load()
    M, stamp, L = state
    _contig(v, "v")
    B, T, H, dv = v.shape
    for name, t in (("alpha", alpha), ("b", b)):
        _contig(t, name, v.dtype, (B, T, H))
    if w is not None:
        _contig(w, "w", v.dtype, v.shape)
    W, R = widx.shape[-1], ridx.shape[-1]
    _contig(widx, "widx", torch.int32, (B, T, H, W))
    _contig(wwt, "wwt", torch.float32, (B, T, H, W))
    _contig(ridx, "ridx", torch.int32, (B, T, H, R))
    _contig(rwt, "rwt", torch.float32, (B, T, H, R))
    _contig(M, "M", torch.float32)
    if M.dim() != 4 or M.shape[0] != B or M.shape[1] != H or M.shape[3] != dv:
        raise ValueError("M must be [B, H, N, d_v]")
    N = M.shape[2]
    _contig(stamp, "stamp", torch.float64, (B, H, dv // 64, N))
    _contig(L, "L", torch.float64, (B, H, dv // 64))
    if o is None:
        o = torch.empty(B, T, H, dv, device=v.device, dtype=torch.float32)
    st = lib.gdn2_sdm_fwd(_ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt),
                          _ptr(M), _ptr(stamp), _ptr(L), _ptr(o), B, T, H, N, dv, W, R, _dtype_code(v),
                          _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_sdm_fwd", st)
    return o


def sdm_fold(state, *, stream=None):
    """Brings the memory up to date (gdn2_sdm_fold): afterwards state[0] is the memory itself."""
    lib = load()
    M, stamp, L = state
    _contig(M, "M", torch.float32)
    B, H, N, dv = M.shape
    _contig(stamp, "stamp", torch.float64, (B, H, dv // 64, N))
    _contig(L, "L", torch.float64, (B, H, dv // 64))
    st = lib.gdn2_sdm_fold(_ptr(M), _ptr(stamp), _ptr(L), B, H, N, dv, _stream(stream))
    if st != 0:
        raise Gdn2Error("gdn2_sdm_fold", st)
    return M
