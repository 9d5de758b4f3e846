"""GPU parity on the method's own edge cases and at the decode workload's full length.

- Decode: 1000 consecutive in-place steps at B256 H16 d128 (the benchmark's launch: inputs cycle
  through 64 seeded step-sets) with 64 seeded-sampled heads against the oracle chained over the
  same 1000 tokens; one step at B1024 H16 d128 (1 GiB of state, the four-wave launch) on sampled
  heads.
- Special cases of the update rule (page "NVIDIA представила Gated DeltaNet-2 …", paragraph
  "Техническая схема"), each against its closed form computed here in float64, on the
  two-kernel prefill, the single-kernel prefill and the decode step:
    b = w = 0: the state only decays, S_T = Diag(prod alpha) S0, o_t = S0^T (gamma_t * q_t);
    alpha = 1, b = 0: causal linear attention, o_t = S0^T q_t + sum_{j<=t} (q_t . k_j)(w_j * v_j).
- Isolation: a NaN in one head's v leaves every other head's o and state bit-equal to a clean run.
- Range: states far above fp16's largest value (v and S0 times 3e4) and far below its smallest
  normal (times 1e-4) on the bf16 prefill, whose matrix-core operands are fp16.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import banner, normwise_err
from gated_delta_rule_25_amd.inputs import WORKLOADS, make_decode_inputs, make_inputs, scaled

pytestmark = pytest.mark.gpu

TOL32 = 1e-5
TOL16 = 2e-3
NAMES = ("q", "k", "v", "alpha", "b", "w")


def _g():
    import gated_delta_rule_25_amd as g
    return g


def _cuda(ins):
    return {n: (x.cuda() if hasattr(x, "cuda") else x) for n, x in ins.items()}


def _prefill(ins, path):
    d = _cuda(ins)
    g = _g()
    if path == "recurrent":
        out = g.recurrent_fwd(*[d[n] for n in NAMES], d["S0"])
    else:
        out = g.chunk_fwd(*[d[n] for n in NAMES], d["S0"], schedule=path)
    torch.cuda.synchronize()
    return out


# ---- decode at the workload's length and batch ---------------------------------------------

def test_decode_1000_steps_b256_sampled_heads():
    """The decode workload as the benchmark runs it: B256 H16 d128, fp32 state updated in place
    for 1000 steps, inputs cycling through 64 step-sets. 64 sampled heads are checked at every
    step (o) and at the end (state) against the oracle run over the same 1000 tokens."""
    banner("decode 1000 steps B256 H16 d128, 64 sampled heads")
    g = _g()
    B, H, d, steps, pool = 256, 16, 128, 1000, 64
    ins = make_decode_inputs(B, H, d, d, pool, seed=20254, device="cuda", generator="torch")
    rng = np.random.Generator(np.random.PCG64(4242))
    flat = rng.choice(B * H, 64, replace=False)
    bs = torch.from_numpy(flat // H).cuda()
    hs = torch.from_numpy(flat % H).cuda()
    S = ins["S0"].clone()
    o = torch.empty(B, H, d, device="cuda")
    xs = [ins[n] for n in NAMES]
    o_sampled = []
    for i in range(steps):
        g.decode_step(*[x[i % pool] for x in xs], S, o=o)
        o_sampled.append(o[bs, hs].clone())
    torch.cuda.synchronize()
    got_o = torch.stack(o_sampled, 1)  # [64, steps, d]
    # the oracle: each sampled head is one sequence of 1000 tokens
    idx = torch.arange(steps) % pool
    sub = {n: ins[n][:, bs, hs].cpu()[idx][:, :, None].transpose(0, 1).contiguous() for n in NAMES}
    S0 = ins["S0"][bs, hs].cpu()[:, None]
    o_ref, S_ref = oracle.forward(*[sub[n] for n in NAMES], S0)
    eo = normwise_err(got_o, o_ref[:, :, 0])
    es = normwise_err(S[bs, hs], S_ref[:, 0])
    worst = max(normwise_err(got_o[i], o_ref[i, :, 0]) for i in range(64))
    print(f"  o err {eo:.2e} (worst head {worst:.2e})  S err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32 and worst <= TOL32, (eo, es, worst)


def test_decode_b1024_one_step_sampled_heads():
    """B1024 H16 d128: 1 GiB of fp32 state, past the Infinity Cache, which the launch serves with
    four-wave workgroups; 128 sampled heads against the oracle."""
    banner("decode B1024 H16 d128 one step, 128 sampled heads")
    g = _g()
    B, H, d = 1024, 16, 128
    ins = make_decode_inputs(B, H, d, d, 1, seed=20255, device="cuda", generator="torch")
    S = ins["S0"].clone()
    o = g.decode_step(*[ins[n][0] for n in NAMES], S)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(77))
    flat = rng.choice(B * H, 128, replace=False)
    bs, hs = torch.from_numpy(flat // H).cuda(), torch.from_numpy(flat % H).cuda()
    xs = [ins[n][0][bs, hs][:, None].cpu() for n in NAMES]  # [128, 1, d] = B 128, H 1
    o_ref, S_ref = oracle.decode_step(*xs, ins["S0"][bs, hs][:, None].cpu())
    eo, es = normwise_err(o[bs, hs][:, None], o_ref), normwise_err(S[bs, hs][:, None], S_ref)
    print(f"  o err {eo:.2e}  S err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32, (eo, es)
    # every state of the batch moved (no workgroup skipped): S differs from S0 in every head
    moved = (S != ins["S0"]).flatten(2).any(-1)
    assert bool(moved.all())


# ---- closed forms ----------------------------------------------------------------------------

def _f64(x):
    return x.double().numpy() if hasattr(x, "double") else np.asarray(x, np.float64)


def _pure_decay(ins):
    q, a, S0 = _f64(ins["q"]), _f64(ins["alpha"]), _f64(ins["S0"])
    gam = np.cumprod(a, axis=1)  # gamma_t = prod_{s<=t} alpha_s, [B, T, H, dk]
    o = np.einsum("bthi,bhij->bthj", gam * q, S0)
    return o, gam[:, -1][..., None] * S0


def _linear_attention(ins):
    q, k, v, w, S0 = (_f64(ins[n]) for n in ("q", "k", "v", "w", "S0"))
    u = w * v
    scores = np.einsum("bthi,bshi->bhts", q, k)
    T = q.shape[1]
    scores = scores * np.tril(np.ones((T, T)))
    o = np.einsum("bhts,bshj->bthj", scores, u) + np.einsum("bthi,bhij->bthj", q, S0)
    return o, S0 + np.einsum("bthi,bthj->bhij", k, u)


PATHS = ["split", "fused", "recurrent"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("d", [64, 128])
def test_pure_decay_closed_form(path, d):
    banner(f"pure decay (b = w = 0) path={path} d={d}")
    ins = make_inputs(scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=3, d_k=d, d_v=d))
    ins["b"] = torch.zeros_like(ins["b"])
    ins["w"] = torch.zeros_like(ins["w"])
    o_ref, S_ref = _pure_decay(ins)
    o, S_T = _prefill(ins, path)
    tol = TOL32 if path == "recurrent" else TOL16
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("d", [64, 128])
def test_linear_attention_closed_form(path, d):
    banner(f"linear attention (alpha = 1, b = 0) path={path} d={d}")
    ins = make_inputs(scaled(WORKLOADS["prefill_1p3b"], B=2, T=150, H=3, d_k=d, d_v=d))
    ins["alpha"] = torch.ones_like(ins["alpha"])
    ins["b"] = torch.zeros_like(ins["b"])
    o_ref, S_ref = _linear_attention(ins)
    o, S_T = _prefill(ins, path)
    tol = TOL32 if path == "recurrent" else TOL16
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


def test_decode_special_cases_closed_form():
    """Decode steps with b = w = 0 (pure decay) and with alpha = 1, b = 0 (linear attention)."""
    banner("decode pure decay and linear attention, 5 steps")
    g = _g()
    B, H, d, steps = 3, 4, 128, 5
    for case in ("decay", "linear"):
        ins = make_decode_inputs(B, H, d, d, steps, seed=31)
        if case == "decay":
            ins["b"] = torch.zeros_like(ins["b"])
            ins["w"] = torch.zeros_like(ins["w"])
        else:
            ins["alpha"] = torch.ones_like(ins["alpha"])
            ins["b"] = torch.zeros_like(ins["b"])
        tok = {n: ins[n].transpose(0, 1).contiguous() for n in NAMES}  # [B, steps, H, d]
        tok["S0"] = ins["S0"]
        o_ref, S_ref = (_pure_decay if case == "decay" else _linear_attention)(tok)
        S = ins["S0"].clone().cuda()
        os_ = []
        for t in range(steps):
            os_.append(g.decode_step(*[ins[n][t].cuda() for n in NAMES], S))
        torch.cuda.synchronize()
        got = torch.stack(os_, 1)
        eo, es = normwise_err(got, o_ref), normwise_err(S, S_ref)
        print(f"  {case}: o err {eo:.2e}  S err {es:.2e}", flush=True)
        assert eo <= TOL32 and es <= TOL32, (case, eo, es)


# ---- NaN isolation ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["split", "fused", "decode"])
def test_nan_in_one_head_stays_in_that_head(path):
    banner(f"NaN isolation path={path}")
    g = _g()
    bad_b, bad_h = 1, 2
    if path == "decode":
        ins = make_decode_inputs(3, 4, 128, 128, 1, seed=12)
        step = {n: ins[n][0].cuda() for n in NAMES}
        S_clean, S_nan = ins["S0"].clone().cuda(), ins["S0"].clone().cuda()
        o_clean = g.decode_step(*[step[n] for n in NAMES], S_clean)
        step["v"] = step["v"].clone()
        step["v"][bad_b, bad_h, 5] = float("nan")
        o_nan = g.decode_step(*[step[n] for n in NAMES], S_nan)
        torch.cuda.synchronize()
        o_clean, o_nan = o_clean[:, None], o_nan[:, None]  # [B, 1, H, d] like a prefill
    else:
        ins = _cuda(make_inputs(scaled(WORKLOADS["prefill_1p3b"], B=2, T=150, H=3)))
        o_clean, S_clean = g.chunk_fwd(*[ins[n] for n in NAMES], ins["S0"], schedule=path)
        v = ins["v"].clone()
        v[bad_b, 70, bad_h, 5] = float("nan")
        o_nan, S_nan = g.chunk_fwd(*[ins[n] for n in NAMES[:2]], v, *[ins[n] for n in NAMES[3:]], ins["S0"],
                                   schedule=path)
        torch.cuda.synchronize()
    B, H = S_clean.shape[:2]
    assert bool(torch.isnan(o_nan[bad_b, :, bad_h]).any()), "the NaN did not reach its own head"
    for b in range(B):
        for h in range(H):
            if (b, h) == (bad_b, bad_h):
                continue
            assert torch.equal(o_nan[b, :, h], o_clean[b, :, h]), (b, h)
            assert torch.equal(S_nan[b, h], S_clean[b, h]), (b, h)


# ---- range of the fp16 matrix-core operands ----------------------------------------------------

RANGE_CASES = [
    ("large_3e4", 3e4, scaled(WORKLOADS["prefill_1p3b"], B=2, T=300, H=3)),
    ("small_1e-4", 1e-4, scaled(WORKLOADS["prefill_1p3b"], B=2, T=300, H=3)),
    ("large_slow_decay", 3e4, scaled(WORKLOADS["long_prefill"], B=1, T=700, H=2)),
    ("large_d64", 3e4, scaled(WORKLOADS["prefill_1p3b"], B=1, T=200, H=2, d_k=64, d_v=64)),
    ("large_gdn", 3e4, scaled(WORKLOADS["gdn_scalar"], B=1, T=200, H=2)),
]


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("name,scale,wl", RANGE_CASES, ids=[c[0] for c in RANGE_CASES])
def test_state_range_beyond_fp16(name, scale, wl, schedule):
    """v and S0 scaled so the state and o lie far outside fp16's normal range (|S| up to about
    1e5, or about 1e-5); bf16 represents them, and the result must stay within the bf16 bar."""
    banner(f"state range {name} schedule={schedule}")
    ins = make_inputs(wl)
    ins["v"] = (ins["v"].float() * scale).to(torch.bfloat16)
    ins["S0"] = ins["S0"] * scale
    a, b, w = ins["alpha"], ins["b"], ins["w"]
    if ins.get("alpha_scalar") or ins.get("beta_scalar"):
        a, b, w = oracle.broadcast_gates(a, b, w, wl.d_k, wl.d_v, alpha_scalar=ins["alpha_scalar"],
                                         beta_scalar=ins["beta_scalar"])
    o_ref, S_ref = oracle.forward(ins["q"], ins["k"], ins["v"], a, b, w, ins["S0"])
    d = _cuda(ins)
    o, S_T = _g().chunk_fwd(*[d[n] for n in NAMES], d["S0"], schedule=schedule)
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  max|S| {np.abs(S_ref).max():.3g}  o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= TOL16 and es <= TOL16, (eo, es)
