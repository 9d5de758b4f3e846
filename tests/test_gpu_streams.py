"""Every entry point runs on the stream it is given: inputs written on a side stream, behind a
long-running kernel on that stream, are read only after those writes, and the results equal the
default-stream results bit for bit (the kernels are deterministic)."""
import pytest
import torch

from parity import banner
from gated_delta_rule_25_amd.inputs import (WORKLOADS, make_cotangents, make_inputs, make_packed_cotangents,
                                            make_packed_inputs, scaled)

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "alpha", "b", "w")


def _g():
    import gated_delta_rule_25_amd as g
    return g


def _side_copies(src, stream):
    """Copies of the device tensors in src made on `stream` after a long matrix product there."""
    with torch.cuda.stream(stream):
        a = torch.randn(4096, 4096, device="cuda")
        for _ in range(4):
            a = a @ a / 64.0  # keeps the stream busy for a while before the copies
        out = {n: (x.clone() if torch.is_tensor(x) else x) for n, x in src.items()}
    return out, a


def test_entry_points_follow_the_given_stream():
    banner("streams: chunk_fwd, chunk_fwd_varlen, chunk_bwd, chunk_bwd_varlen, decode_step, rmsnorm on a side stream")
    g = _g()
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=300, H=4)
    ins = make_inputs(wl)
    cot = make_cotangents(wl)
    d = {n: (ins[n].cuda() if ins[n] is not None else None) for n in NAMES + ("S0",)}
    d.update(dO=cot["dO"].cuda(), dS_T=cot["dS_T"].cuda())
    d.update({n + "1": d[n][:, 0].contiguous() for n in NAMES})  # one decode token
    packed = make_packed_inputs(scaled(wl, H=2), [70, 0, 130, 5], device="cuda")
    pcot = make_packed_cotangents(scaled(wl, H=2), [70, 0, 130, 5], device="cuda")
    packed.update(dO=pcot["dO"], dS_T=pcot["dS_T"])

    def run(x, p, stream):
        o, S = g.chunk_fwd(*(x[n] for n in NAMES), x["S0"], stream=stream)
        ov, Sv = g.chunk_fwd_varlen(*(p[n] for n in NAMES), p["cu_seqlens"], p["S0"], stream=stream)
        gr = g.chunk_bwd(*(x[n] for n in NAMES), x["S0"], x["dO"], x["dS_T"], stream=stream)
        Sd = x["S0"].clone() if stream is None else None
        if stream is not None:
            with torch.cuda.stream(stream):
                Sd = x["S0"].clone()
        od = g.decode_step(*(x[n + "1"] for n in NAMES), Sd, stream=stream)
        gv = g.chunk_bwd_varlen(*(p[n] for n in NAMES), p["cu_seqlens"], p["S0"], p["dO"], p["dS_T"],
                                stream=stream)
        y = g.rmsnorm_fwd(x["dO"], None, eps=1e-6, stream=stream)
        gn = g.rmsnorm_bwd(x["dO"], None, x["dO"], eps=1e-6, stream=stream)
        return ([o, S, ov, Sv, od, Sd, y, gn["dx"], gn["dweight"]] + [gr[k] for k in sorted(gr)]
                + [gv[k] for k in sorted(gv)])

    ref = run(d, packed, None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    xd, _ = _side_copies(d, s)
    xp, _ = _side_copies(packed, s)
    got = run(xd, xp, s)
    s.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), i
