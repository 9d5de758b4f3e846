"""GPU parity: the fused prologue (GDN2_QK_L2NORM, GDN2_GATE_LOGITS) against the oracle.

Raw inputs (unnormalised q, k; gate pre-activations) go to the kernels with the flags set; the
oracle applies its own prologue (oracle.prologue: x / max(|x|, 1e-12) and 1 / (1 + e^-x) in
float64) and then the recurrence. Bars as for the same paths without the prologue: 2e-3 (bf16
inputs on the two-kernel prefill), 1e-5 (fp32 inputs on it, and the fp32 token-by-token
prefill and decode step).
"""
import pytest
import torch

import oracle
from parity import banner, normwise_err
from gated_delta_rule_25_amd.inputs import WORKLOADS, make_prologue_inputs, scaled

pytestmark = pytest.mark.gpu

TOL16, TOL32 = 2e-3, 1e-5


def _g():
    import gated_delta_rule_25_amd as g
    return g


def _oracle(ins, l2norm, gate_logits):
    q, k, a, b, w = oracle.prologue(ins["q"], ins["k"], ins["alpha"], ins["b"], ins["w"],
                                    l2norm=l2norm, gate_logits=gate_logits)
    dk, dv = q.shape[-1], ins["v"].shape[-1]
    if ins["alpha_scalar"] or ins["beta_scalar"]:
        a, b, w = oracle.broadcast_gates(a, b, w, dk, dv, alpha_scalar=ins["alpha_scalar"],
                                         beta_scalar=ins["beta_scalar"])
    return oracle.forward(q, k, ins["v"], a, b, w, ins["S0"])


def _cuda(ins):
    return {n: (x.cuda() if hasattr(x, "cuda") else x) for n, x in ins.items()}


CASES = [
    ("bf16_d128_both", scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=3), True, True, TOL16),
    ("bf16_d128_l2norm", scaled(WORKLOADS["prefill_1p3b"], B=1, T=130, H=2), True, False, TOL16),
    ("bf16_d128_logits", scaled(WORKLOADS["prefill_1p3b"], B=1, T=130, H=2), False, True, TOL16),
    ("bf16_d64_both", scaled(WORKLOADS["prefill_1p3b"], B=2, T=150, H=2, d_k=64, d_v=64), True, True, TOL16),
    ("bf16_gdn_both", scaled(WORKLOADS["gdn_scalar"], B=1, T=200, H=2), True, True, TOL16),
    ("bf16_kda_both", scaled(WORKLOADS["kda_scalar"], B=1, T=200, H=2), True, True, TOL16),
    ("fp32_d32_both", scaled(WORKLOADS["tiny_fp32"], B=1, T=150, H=2, s0_std=0.1), True, True, TOL32),
    # fp32 at d = 64 and 128 on the two-kernel path (one block buffer; v, w in registers at 128)
    ("fp32_d128_both", scaled(WORKLOADS["prefill_1p3b"], B=1, T=150, H=2, dtype="fp32"), True, True, TOL32),
    ("fp32_d128_kda_both", scaled(WORKLOADS["kda_scalar"], B=1, T=100, H=2, dtype="fp32"), True, True, TOL32),
    ("fp32_d64_logits", scaled(WORKLOADS["prefill_1p3b"], B=2, T=90, H=2, d_k=64, d_v=64, dtype="fp32"), False, True,
     TOL32),
]


def _inputs(wl, l2n, gl):
    """Raw inputs for the steps the kernel does; the step it does not do is applied here (in
    float64, then rounded to the input dtype), so every case runs on valid gates and keys."""
    ins = make_prologue_inputs(wl)
    if l2n and gl:
        return ins
    q, k, a, b, w = oracle.prologue(ins["q"], ins["k"], ins["alpha"], ins["b"], ins["w"],
                                    l2norm=not l2n, gate_logits=not gl)
    dt = ins["q"].dtype
    t = lambda x: None if x is None else torch.from_numpy(x).to(dt)
    ins.update(q=t(q), k=t(k), alpha=t(a), b=t(b), w=t(w))
    return ins


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("name,wl,l2n,gl,tol", CASES, ids=[c[0] for c in CASES])
def test_chunk_prologue_matches_oracle(name, wl, l2n, gl, tol, schedule):
    if schedule == "fused" and wl.dtype == "fp32":
        pytest.skip("without a workspace fp32 inputs run the single kernel (d <= 64), which takes no "
                    "prologue flags; fp32 at d = 128 runs with a workspace only")
    banner(f"prologue chunk {name} l2norm={l2n} logits={gl} schedule={schedule} {wl}")
    ins = _inputs(wl, l2n, gl)
    o_ref, S_ref = _oracle(ins, l2n, gl)
    d = _cuda(ins)
    o, S_T = _g().chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"],
                            l2norm=l2n, gate_logits=gl, schedule=schedule)
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  {name}: o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("gates", ["general", "gdn"])
def test_recurrent_prologue_matches_oracle(gates):
    wl = scaled(WORKLOADS["prefill_1p3b" if gates == "general" else "gdn_scalar"], B=1, T=90, H=2)
    banner(f"prologue recurrent {gates} {wl}")
    ins = make_prologue_inputs(wl)
    o_ref, S_ref = _oracle(ins, True, True)
    d = _cuda(ins)
    o, S_T = _g().recurrent_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"],
                                l2norm=True, gate_logits=True)
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  recurrent {gates}: o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32, (eo, es)


def test_decode_prologue_matches_oracle():
    wl = scaled(WORKLOADS["prefill_1p3b"], B=4, T=1, H=3)
    banner(f"prologue decode {wl}")
    ins = make_prologue_inputs(wl)
    o_ref, S_ref = _oracle(ins, True, True)
    d = _cuda(ins)
    S = d["S0"].clone()
    o = _g().decode_step(*(d[n][:, 0] for n in ("q", "k", "v", "alpha", "b", "w")), S,
                         l2norm=True, gate_logits=True)
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_ref[:, 0]), normwise_err(S, S_ref)
    print(f"  decode: o err {eo:.2e}  S err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32, (eo, es)


def test_single_kernel_path_refuses_the_prologue():
    """fp32 inputs without a workspace run the single kernel, which does not take the flags."""
    g = _g()
    wl = scaled(WORKLOADS["tiny_fp32"], B=1, T=64, H=1)
    d = _cuda(make_prologue_inputs(wl))
    with pytest.raises(g.Gdn2Error) as e:
        g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"], schedule="fused", l2norm=True)
    assert e.value.status == 3
