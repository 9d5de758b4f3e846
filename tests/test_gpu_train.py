"""GPU parity: a training step through gdn2_chunk_fwd_save and gdn2_chunk_bwd_saved.

The forward that saves computes o and S_T and leaves in the backward workspace the operand blocks,
the chunk-start states and the D', Delta rows; the backward then reads them instead of recomputing
the forward. o and S_T are checked against the fp64 oracle's forward at the bf16 forward's bar
(normwise 2e-3), the gradients against the oracle's backward at the backward's bar (2e-3). The
saves are made by the same arithmetic as gdn2_chunk_bwd's own recomputation (the same matrix-core
products in the same order on the same operands), so the gradients of the two backward calls
must agree to the bit; gate forms and prologue flags are checked that way against gdn2_chunk_bwd,
whose own parity with the oracle the backward tests establish.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import banner, normwise_err
from gated_delta_rule_25_amd.inputs import WORKLOADS, make_cotangents, make_inputs, make_prologue_inputs, scaled

pytestmark = pytest.mark.gpu

TOL = 2e-3
NAMES = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")


def _g():
    import gated_delta_rule_25_amd as g
    return g


def _cuda(x):
    return None if x is None else x.cuda()


def _step(ins, cot, l2n=False, gl=False):
    """(o, S_T) and the gradients through the saving forward and the saved backward, and the
    gradients of gdn2_chunk_bwd (recomputing) on the same inputs."""
    g = _g()
    d = {n: _cuda(ins[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    args = [d[n] for n in ("q", "k", "v", "alpha", "b", "w", "S0")]
    o, S_T, ws = g.chunk_fwd_save(*args, l2norm=l2n, gate_logits=gl)
    dO, dS = _cuda(cot["dO"]), _cuda(cot["dS_T"])
    saved = g.chunk_bwd(*args, dO, dS, l2norm=l2n, gate_logits=gl, saved=ws)
    again = g.chunk_bwd(*args, dO, dS, l2norm=l2n, gate_logits=gl, saved=ws)
    recomputed = g.chunk_bwd(*args, dO, dS, l2norm=l2n, gate_logits=gl)
    torch.cuda.synchronize()
    return o, S_T, saved, again, recomputed


def _same(a, b, label):
    for n in a:
        assert torch.equal(a[n], b[n]), f"{label}: {n} differs (max {(a[n] - b[n]).abs().max().item():.3e})"


CASES = [
    ("d128_ragged", scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=3)),
    ("d64_ragged", scaled(WORKLOADS["prefill_1p3b"], B=2, T=150, H=2, d_k=64, d_v=64)),
    ("d32_ragged", scaled(WORKLOADS["prefill_1p3b"], B=1, T=100, H=2, d_k=32, d_v=32)),
    ("d128_T1", scaled(WORKLOADS["prefill_1p3b"], B=1, T=1, H=2)),
    ("d128_T64", scaled(WORKLOADS["prefill_1p3b"], B=1, T=64, H=2)),
    ("d128_strong_decay", scaled(WORKLOADS["prefill_1p3b"], B=1, T=260, H=3, alpha_mu=-2.0)),
    ("d128_zero_s0", scaled(WORKLOADS["prefill_1p3b"], B=1, T=300, H=2, s0_std=0.0)),
]


@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_train_step_matches_oracle(name, wl):
    banner(f"train step {name} {wl}")
    ins = make_inputs(wl)
    cot = make_cotangents(wl)
    o, S_T, saved, again, recomputed = _step(ins, cot)
    x = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    o_ref, S_ref = oracle.forward(*x, S0=ins["S0"])
    ref = oracle.backward(*x, ins["S0"], cot["dO"], cot["dS_T"])
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    errs = {n: normwise_err(saved[n], ref[n]) for n in NAMES}
    print(f"  o {eo:.2e}  S_T {es:.2e}  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert eo <= TOL and es <= TOL, (eo, es)
    assert all(e <= TOL for e in errs.values()), errs
    _same(saved, recomputed, "saved vs recomputed backward")
    _same(saved, again, "second call on the same saves")


@pytest.mark.parametrize("gates", ["gdn", "kda"])
def test_train_step_scalar_gates(gates):
    wl = scaled(WORKLOADS[f"{gates}_scalar"], B=2, T=150, H=2)
    banner(f"train step scalar gates {gates} {wl}")
    ins = make_inputs(wl)
    cot = make_cotangents(wl)
    o, S_T, saved, again, recomputed = _step(ins, cot)
    g = _g()
    o_r, S_r = g.chunk_fwd(*[_cuda(ins[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")])
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_r.cpu()), normwise_err(S_T, S_r.cpu())
    print(f"  o vs chunk_fwd {eo:.2e}  S_T {es:.2e}", flush=True)
    assert eo <= TOL and es <= TOL
    assert "dw" not in saved
    _same(saved, recomputed, "saved vs recomputed backward")
    _same(saved, again, "second call on the same saves")


@pytest.mark.parametrize("l2n,gl", [(True, True), (True, False), (False, True)])
def test_train_step_prologue(l2n, gl):
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=150, H=2)
    banner(f"train step prologue l2norm={l2n} logits={gl} {wl}")
    ins = make_prologue_inputs(wl)
    if not (l2n and gl):  # the step the kernels do not take is applied here (float64, then bf16)
        q, k, a, b, w = oracle.prologue(ins["q"], ins["k"], ins["alpha"], ins["b"], ins["w"],
                                        l2norm=not l2n, gate_logits=not gl)
        t = lambda x: None if x is None else torch.from_numpy(np.asarray(x)).to(torch.bfloat16)
        ins.update(q=t(q), k=t(k), alpha=t(a), b=t(b), w=t(w))
    cot = make_cotangents(wl)
    o, S_T, saved, again, recomputed = _step(ins, cot, l2n, gl)
    g = _g()
    o_r, S_r = g.chunk_fwd(*[_cuda(ins[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")], l2norm=l2n,
                           gate_logits=gl)
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_r.cpu()), normwise_err(S_T, S_r.cpu())
    print(f"  o vs chunk_fwd {eo:.2e}  S_T {es:.2e}", flush=True)
    assert eo <= TOL and es <= TOL
    _same(saved, recomputed, "saved vs recomputed backward")


def test_train_step_full_size_sampled_heads():
    """At B8 H16 T4096 d128 (the backward benchmark's launch): o of two sampled (b, h) sequences
    against the oracle's forward of those sequences alone, and the saved backward equal to the
    recomputing one everywhere."""
    banner("train step full size B8 H16 T4096, heads (0, 0) and (7, 13)")
    from gated_delta_rule_25_amd.inputs import make_inputs_torch
    wl = WORKLOADS["prefill_1p3b"]
    ins = make_inputs_torch(wl, device="cuda")
    cot = make_cotangents(wl, device="cuda")
    g = _g()
    args = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w", "S0")]
    o, S_T, ws = g.chunk_fwd_save(*args)
    saved = g.chunk_bwd(*args, cot["dO"], cot["dS_T"], saved=ws)
    del ws
    recomputed = g.chunk_bwd(*args, cot["dO"], cot["dS_T"])
    torch.cuda.synchronize()
    _same(saved, recomputed, "saved vs recomputed backward")
    del recomputed
    for bb, hh in ((0, 0), (7, 13)):
        sl = lambda x: x[bb:bb + 1, :, hh:hh + 1].cpu()
        o_ref, S_ref = oracle.forward(*[sl(ins[n]) for n in ("q", "k", "v", "alpha", "b", "w")],
                                      S0=ins["S0"][bb:bb + 1, hh:hh + 1].cpu())
        eo = normwise_err(o[bb:bb + 1, :, hh:hh + 1], o_ref)
        es = normwise_err(S_T[bb:bb + 1, hh:hh + 1], S_ref)
        print(f"  head ({bb}, {hh}): o {eo:.2e}  S_T {es:.2e}", flush=True)
        assert eo <= TOL and es <= TOL, (eo, es)


def test_train_step_no_tokens():
    banner("train step, T = 0")
    g = _g()
    S0 = torch.randn(2, 3, 64, 64, device="cuda")
    dS = torch.randn(2, 3, 64, 64, device="cuda")
    e = torch.empty(2, 0, 3, 64, dtype=torch.bfloat16, device="cuda")
    o, S_T, ws = g.chunk_fwd_save(e, e, e, e, e, e, S0)
    out = g.chunk_bwd(e, e, e, e, e, e, S0, torch.empty(2, 0, 3, 64, device="cuda"), dS, saved=ws)
    torch.cuda.synchronize()
    assert ws is None and o.numel() == 0
    assert torch.equal(S_T, S0) and torch.equal(out["dS0"], dS)


# ---- packed batches: gdn2_chunk_fwd_varlen_save + gdn2_chunk_bwd_varlen_saved ----------------

VAR_CASES = [
    ("d128_mix", scaled(WORKLOADS["prefill_1p3b"], H=2), [0, 1, 63, 64, 65, 200, 0, 130, 17, 257], False, False),
    ("d64", scaled(WORKLOADS["prefill_1p3b"], H=3, d_k=64, d_v=64), [5, 0, 128, 300], False, False),
    ("d32", scaled(WORKLOADS["prefill_1p3b"], H=2, d_k=32, d_v=32), [70, 1, 190], False, False),
    ("gdn", scaled(WORKLOADS["gdn_scalar"], H=2), [100, 64, 0, 3], False, False),
    ("kda_prologue", scaled(WORKLOADS["kda_scalar"], H=2), [3, 150, 0], True, True),
    ("general_prologue", scaled(WORKLOADS["prefill_1p3b"], H=2), [70, 0, 129, 5], True, True),
]


@pytest.mark.parametrize("name,wl,lengths,l2n,gl", VAR_CASES, ids=[c[0] for c in VAR_CASES])
def test_train_step_packed(name, wl, lengths, l2n, gl):
    """The packed forward that saves against gdn2_chunk_fwd_varlen (o and S_T within the bf16 bar;
    each sequence's o against the oracle's forward of it alone where no prologue flag applies),
    and the saved packed backward bit-equal to gdn2_chunk_bwd_varlen."""
    from gated_delta_rule_25_amd.inputs import make_packed_cotangents, make_packed_inputs
    banner(f"train step packed {name} lengths={lengths} {wl}")
    g = _g()
    ins = make_packed_inputs(wl, lengths, raw=l2n or gl)
    cot = make_packed_cotangents(wl, lengths)
    names = ("q", "k", "v", "alpha", "b", "w")
    x = [_cuda(ins[n]) for n in names]
    cu = ins["cu_seqlens"].cuda()
    S0 = _cuda(ins["S0"])
    dO, dS = _cuda(cot["dO"]), _cuda(cot["dS_T"])
    o, S_T, ws = g.chunk_fwd_varlen_save(*x, cu, S0, l2norm=l2n, gate_logits=gl)
    saved = g.chunk_bwd_varlen(*x, cu, S0, dO, dS, l2norm=l2n, gate_logits=gl, saved=ws)
    again = g.chunk_bwd_varlen(*x, cu, S0, dO, dS, l2norm=l2n, gate_logits=gl, saved=ws)
    recomputed = g.chunk_bwd_varlen(*x, cu, S0, dO, dS, l2norm=l2n, gate_logits=gl)
    o_r, S_r = g.chunk_fwd_varlen(*x, cu, S0, l2norm=l2n, gate_logits=gl)
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_r), normwise_err(S_T, S_r)
    print(f"  o vs chunk_fwd_varlen {eo:.2e}  S_T {es:.2e}", flush=True)
    assert eo <= TOL and es <= TOL, (eo, es)
    _same(saved, recomputed, "saved vs recomputed packed backward")
    _same(saved, again, "second call on the same saves")
    if not (l2n or gl or ins["alpha_scalar"] or ins["beta_scalar"]):
        bounds = ins["cu_seqlens"].tolist()
        for s in range(len(lengths)):
            lo, hi = bounds[s], bounds[s + 1]
            if hi == lo:
                assert torch.equal(S_T[s].cpu(), ins["S0"][s]), s
                continue
            o_ref, S_ref = oracle.forward(*[ins[n][lo:hi].unsqueeze(0) for n in names], S0=ins["S0"][s:s + 1])
            e1, e2 = normwise_err(o[lo:hi].unsqueeze(0), o_ref), normwise_err(S_T[s:s + 1], S_ref)
            assert e1 <= TOL and e2 <= TOL, (s, e1, e2)


def test_train_step_packed_no_rows():
    banner("train step packed, T_total = 0")
    g = _g()
    S0 = torch.randn(3, 2, 64, 64, device="cuda")
    e = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    o, S_T, ws = g.chunk_fwd_varlen_save(e, e, e, e, e, e, cu, S0)
    torch.cuda.synchronize()
    assert ws is None and o.numel() == 0 and torch.equal(S_T, S0)
