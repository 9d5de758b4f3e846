"""Error measures for GPU-vs-oracle parity tests.

Normwise relative error: max |x - y| / max |y| over one output tensor. Elementwise relative
error is ill-posed where the reference is near zero; the normwise form bounds every element's
error relative to the tensor's scale.
"""
import numpy as np


def to64(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def normwise_err(x, ref) -> float:
    x, ref = to64(x), to64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    scale = np.abs(ref).max()
    d = np.abs(x - ref).max()
    return float(d / scale) if scale > 0 else float(d)


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
