"""GPU parity: the chunkwise (C = 64) prefill kernel against the fp64 oracle.

Bars (normwise max relative error, see parity.py): <= 1e-5 for fp32 inputs (fp32 matrix-core
operands throughout) and <= 2e-3 for bf16 inputs (fp16 operands, fp32 accumulation and state),
on o and on the final state. Sizes span several chunks and a ragged last chunk.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import banner, normwise_err
from gated_delta_rule_25_amd.inputs import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

TOL32 = 1e-5
TOL16 = 2e-3


def _g():
    import gated_delta_rule_25_amd as g
    return g


def _oracle(ins):
    a, b, w = ins["alpha"], ins["b"], ins["w"]
    dk, dv = ins["q"].shape[-1], ins["v"].shape[-1]
    if ins.get("alpha_scalar") or ins.get("beta_scalar"):
        a, b, w = oracle.broadcast_gates(a, b, w, dk, dv, alpha_scalar=ins["alpha_scalar"],
                                         beta_scalar=ins["beta_scalar"])
    return oracle.forward(ins["q"], ins["k"], ins["v"], a, b, w, ins["S0"])


def _cuda(ins):
    return {n: (x.cuda() if hasattr(x, "cuda") else x) for n, x in ins.items()}


def _run(ins, **kw):
    d = _cuda(ins)
    out = _g().chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"], **kw)
    torch.cuda.synchronize()
    return out


def _check(name, ins, tol, schedule="split"):
    o_ref, S_ref = _oracle(ins)
    o, S_T = _run(ins, schedule=schedule)
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  {name} ({schedule}): o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


# split: two kernels through operand blocks (with a workspace); fused: no workspace (the fused
# kernel, or the single kernel for sizes it does not take)
SCHEDULES = ["split", "fused"]


FP32_CASES = [
    ("tiny_fp32_full", WORKLOADS["tiny_fp32"]),
    ("fp32_d32_ragged_s0", scaled(WORKLOADS["tiny_fp32"], B=2, T=150, H=3, s0_std=0.1)),
    ("fp32_d64_ragged", scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=2, d_k=64, d_v=64,
                               dtype="fp32")),
    ("fp32_d64_gdn", scaled(WORKLOADS["gdn_scalar"], B=1, T=130, H=2, d_k=64, d_v=64,
                            dtype="fp32")),
    ("fp32_d32_kda", scaled(WORKLOADS["kda_scalar"], B=1, T=96, H=3, d_k=32, d_v=32,
                            dtype="fp32")),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,wl", FP32_CASES, ids=[c[0] for c in FP32_CASES])
def test_chunk_fp32_matches_oracle(name, wl, schedule):
    banner(f"chunk fp32 {name} schedule={schedule} {wl}")
    _check(name, make_inputs(wl), TOL32, schedule)


# fp32 at d = 128 runs the two-kernel path only (fp32 operand blocks, one block buffer, v and w
# loaded into registers): ragged T, S0 = 0, the scalar gate forms, strong decay, a single token,
# and several rounds of a small workspace ring.
FP32_D128_CASES = [
    ("fp32_d128_ragged", scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=2, dtype="fp32")),
    ("fp32_d128_zero_s0", scaled(WORKLOADS["prefill_1p3b"], B=1, T=130, H=3, s0_std=0.0, dtype="fp32")),
    ("fp32_d128_gdn", scaled(WORKLOADS["gdn_scalar"], B=1, T=150, H=2, dtype="fp32")),
    ("fp32_d128_kda", scaled(WORKLOADS["kda_scalar"], B=1, T=100, H=2, dtype="fp32")),
    ("fp32_d128_strong_decay", scaled(WORKLOADS["prefill_1p3b"], B=1, T=190, H=2, alpha_mu=-2.0, dtype="fp32")),
    ("fp32_d128_T1", scaled(WORKLOADS["prefill_1p3b"], B=2, T=1, H=2, dtype="fp32")),
]


@pytest.mark.parametrize("name,wl", FP32_D128_CASES, ids=[c[0] for c in FP32_D128_CASES])
def test_chunk_fp32_d128_matches_oracle(name, wl):
    banner(f"chunk fp32 d128 {name} {wl}")
    _check(name, make_inputs(wl), TOL32, "split")


def test_chunk_fp32_d128_small_ring():
    banner("chunk fp32 d128, workspace ring of 2 chunk slots")
    g = _g()
    wl = scaled(WORKLOADS["prefill_1p3b"], B=1, T=300, H=2, dtype="fp32")
    ins = make_inputs(wl)
    d = _cuda(ins)
    B, T, H, dk = d["q"].shape
    per_chunk = g.chunk_fwd_workspace_bytes(B, 64, H, dk, dk, dtype=torch.float32) - B * H * dk * dk * 4
    ws = torch.empty(B * H * dk * dk * 4 + 2 * per_chunk, dtype=torch.uint8, device="cuda")  # 2 of 5 slots
    o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"], workspace=ws,
                         schedule="split")
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(ins)
    eo, es = normwise_err(o, o_ref), normwise_err(S_T, S_ref)
    print(f"  fp32 d128 ring of 2: o err {eo:.2e}  S_T err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32


BF16_CASES = [
    ("bf16_d128_ragged", scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=3)),
    ("bf16_d128_T1", scaled(WORKLOADS["prefill_1p3b"], B=1, T=1, H=2)),
    ("bf16_d128_T63", scaled(WORKLOADS["prefill_1p3b"], B=1, T=63, H=2)),
    ("bf16_d128_T64", scaled(WORKLOADS["prefill_1p3b"], B=1, T=64, H=2)),
    ("bf16_d128_T65", scaled(WORKLOADS["prefill_1p3b"], B=1, T=65, H=2)),
    ("bf16_d128_zero_s0", scaled(WORKLOADS["prefill_1p3b"], B=1, T=300, H=2, s0_std=0.0)),
    ("bf16_d128_slow_decay", scaled(WORKLOADS["long_prefill"], T=1000, H=3)),
    ("bf16_d128_strong_decay", scaled(WORKLOADS["prefill_1p3b"], B=1, T=260, H=3, alpha_mu=-2.0)),
    ("bf16_d64", scaled(WORKLOADS["prefill_1p3b"], B=3, T=190, H=2, d_k=64, d_v=64)),
    ("bf16_d32", scaled(WORKLOADS["prefill_1p3b"], B=2, T=130, H=5, d_k=32, d_v=32)),
    ("bf16_d128_gdn", scaled(WORKLOADS["gdn_scalar"], B=1, T=257, H=3)),
    ("bf16_d128_kda", scaled(WORKLOADS["kda_scalar"], B=1, T=257, H=3)),
    ("bf16_d64_gdn", scaled(WORKLOADS["gdn_scalar"], B=2, T=100, H=2, d_k=64, d_v=64)),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,wl", BF16_CASES, ids=[c[0] for c in BF16_CASES])
def test_chunk_bf16_matches_oracle(name, wl, schedule):
    banner(f"chunk bf16 {name} schedule={schedule} {wl}")
    _check(name, make_inputs(wl), TOL16, schedule)


def test_chunk_zero_tokens_copies_state():
    banner("chunk T=0")
    ins = _cuda(make_inputs(scaled(WORKLOADS["prefill_1p3b"], B=2, T=0, H=3)))
    o, S_T = _g().chunk_fwd(ins["q"], ins["k"], ins["v"], ins["alpha"], ins["b"], ins["w"],
                            ins["S0"])
    torch.cuda.synchronize()
    assert torch.equal(S_T, ins["S0"])


def test_chunk_state_in_place_and_split_invariance():
    """fwd(T1) then fwd(T2) from its state equals fwd(T1 + T2), with S_out aliasing S0."""
    banner("chunk split invariance, in-place state")
    g = _g()
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=2)
    ins = _cuda(make_inputs(wl))
    names = ("q", "k", "v", "alpha", "b", "w")
    o_full, S_full = g.chunk_fwd(*[ins[n] for n in names], ins["S0"])
    S = ins["S0"].clone()
    T1 = 77
    o1, _ = g.chunk_fwd(*[ins[n][:, :T1].contiguous() for n in names], S, S_out=S)
    o2, _ = g.chunk_fwd(*[ins[n][:, T1:].contiguous() for n in names], S, S_out=S)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(make_inputs(wl))
    assert normwise_err(torch.cat([o1, o2], 1), o_ref) <= TOL16
    assert normwise_err(S, S_ref) <= TOL16
    assert normwise_err(S, S_full.double().cpu().numpy()) <= TOL16


def test_chunk_then_decode_equals_longer_prefill():
    banner("chunk(T) + decode == chunk(T+1)")
    g = _g()
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=131, H=2)
    ins = _cuda(make_inputs(wl))
    names = ("q", "k", "v", "alpha", "b", "w")
    o_all, S_all = g.chunk_fwd(*[ins[n] for n in names], ins["S0"])
    o_pre, S = g.chunk_fwd(*[ins[n][:, :-1].contiguous() for n in names], ins["S0"])
    o_last = g.decode_step(*[ins[n][:, -1].contiguous() for n in names], S)
    torch.cuda.synchronize()
    ref = o_all[:, -1].double().cpu().numpy()
    assert normwise_err(o_last, ref) <= TOL16
    assert normwise_err(S, S_all.double().cpu().numpy()) <= TOL16


def test_chunk_is_deterministic():
    banner("chunk bitwise determinism")
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=190, H=3)
    ins = make_inputs(wl)
    o1, S1 = _run(ins)
    o2, S2 = _run(ins)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_chunk_exact_write_invariant():
    """b = 1, q = k with exactly-unit bf16 keys: every o_t equals w_t * v_t (any decay)."""
    banner("chunk exact-write invariant")
    rng = np.random.default_rng(3)
    B, T, H, d = 1, 150, 2, 128
    k = np.zeros((B, T, H, d), np.float32)
    idx = rng.integers(0, d, size=(B, T, H, 4))
    signs = rng.choice([-0.5, 0.5], size=(B, T, H, 4))
    for t in range(T):  # four distinct channels of +-1/2: norm exactly 1
        for h in range(H):
            ch = rng.choice(d, 4, replace=False)
            k[0, t, h, ch] = signs[0, t, h]
    wl = scaled(WORKLOADS["prefill_1p3b"], B=B, T=T, H=H)
    ins = make_inputs(wl)
    kt = torch.from_numpy(k).to(torch.bfloat16)
    ins["k"] = kt
    ins["q"] = kt.clone()
    ins["b"] = torch.ones_like(ins["b"])
    o, _ = _run(ins)
    expect = (ins["w"].double() * ins["v"].double()).numpy()
    assert normwise_err(o, expect) <= TOL16


FULL = [
    ("prefill_1p3b", WORKLOADS["prefill_1p3b"]),
    ("gdn_scalar", WORKLOADS["gdn_scalar"]),
    ("kda_scalar", WORKLOADS["kda_scalar"]),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,wl", FULL, ids=[c[0] for c in FULL])
def test_chunk_full_size_all_heads(name, wl, schedule):
    """The benchmark's launch configuration, B8 H16 T4096 d128, every head against the oracle."""
    banner(f"chunk full {name} schedule={schedule}")
    _check(name, make_inputs(wl), TOL16, schedule)


def test_chunk_split_small_ring():
    """The two-kernel path with a ring of 3 chunk slots (several prep/chain rounds, the state
    carried between rounds) equals the oracle."""
    banner("chunk split, 3-slot ring")
    import gated_delta_rule_25_amd as g
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=450, H=3)
    ins = make_inputs(wl)
    d = _cuda(ins)
    B, T, H, dk = d["q"].shape
    per_chunk = g.chunk_fwd_workspace_bytes(B, 64, H, dk, dk) - B * H * dk * dk * 4
    ws = torch.empty(B * H * dk * dk * 4 + 3 * per_chunk, dtype=torch.uint8, device="cuda")
    o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"],
                         workspace=ws, schedule="split")
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(ins)
    assert normwise_err(o, o_ref) <= TOL16 and normwise_err(S_T, S_ref) <= TOL16


# Long sequences with few (b, h) run the chain in parallel segments (each segment's transition
# from the state recurrence alone, a scan for the segment start states, then all segments at
# once). These sizes are long enough to be segmented; the last segment is ragged.
SEGMENTED = [
    ("seg_bf16_d128", scaled(WORKLOADS["prefill_1p3b"], B=1, T=4100, H=2), TOL16),
    ("seg_bf16_d128_slow_decay", scaled(WORKLOADS["long_prefill"], B=1, T=3000, H=2), TOL16),
    ("seg_bf16_gdn", scaled(WORKLOADS["gdn_scalar"], B=1, T=3000, H=3), TOL16),
    ("seg_bf16_kda", scaled(WORKLOADS["kda_scalar"], B=1, T=2100, H=2), TOL16),
    ("seg_bf16_d64", scaled(WORKLOADS["prefill_1p3b"], B=1, T=2500, H=2, d_k=64, d_v=64), TOL16),
    ("seg_fp32_d32", scaled(WORKLOADS["tiny_fp32"], B=1, T=2100, H=1, s0_std=0.1), TOL32),
    ("seg_fp32_d128", scaled(WORKLOADS["prefill_1p3b"], B=1, T=2100, H=1, dtype="fp32"), TOL32),
    ("seg_fp32_d64", scaled(WORKLOADS["prefill_1p3b"], B=1, T=2100, H=1, d_k=64, d_v=64, dtype="fp32"), TOL32),
    # strong decay: the segments' transitions decay far below fp32's normal range over a segment
    ("seg_bf16_strong_decay", scaled(WORKLOADS["prefill_1p3b"], B=1, T=3000, H=2, alpha_mu=-2.0), TOL16),
]


@pytest.mark.parametrize("name,wl,tol", SEGMENTED, ids=[c[0] for c in SEGMENTED])
def test_chunk_segmented_matches_oracle(name, wl, tol):
    banner(f"chunk segmented {name} {wl}")
    g = _g()
    B, T, H, d = wl.B, wl.T, wl.H, wl.d_k
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    # the workspace query includes the segment buffers exactly when the sizes are segmented
    assert g.chunk_fwd_workspace_bytes(B, T, H, d, d, dtype=dt) > B * H * d * d * 4 + \
        ((T + 63) // 64) * (g.chunk_fwd_workspace_bytes(B, 64, H, d, d, dtype=dt) - B * H * d * d * 4)
    _check(name, make_inputs(wl), tol, "split")


def test_chunk_segmented_in_place_state():
    """Segmented run with S_out aliasing S0, then the next call continues from that state."""
    banner("chunk segmented, in-place state")
    g = _g()
    wl = scaled(WORKLOADS["prefill_1p3b"], B=1, T=4100, H=2)
    ins = make_inputs(wl)
    d = _cuda(ins)
    names = ("q", "k", "v", "alpha", "b", "w")
    S = d["S0"].clone()
    T1 = 2300
    o1, _ = g.chunk_fwd(*[d[n][:, :T1].contiguous() for n in names], S, S_out=S)
    o2, _ = g.chunk_fwd(*[d[n][:, T1:].contiguous() for n in names], S, S_out=S)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(ins)
    assert normwise_err(torch.cat([o1, o2], 1), o_ref) <= TOL16
    assert normwise_err(S, S_ref) <= TOL16


def test_chunk_long_context_sampled_heads():
    """B1 H16 T131072 (the long-context shape, segmented): o and S_T of two heads against the
    oracle over all 131,072 tokens."""
    from gated_delta_rule_25_amd.inputs import make_inputs_torch
    banner("chunk long context, heads 0 and 11")
    g = _g()
    wl = WORKLOADS["long_prefill"]
    ins = make_inputs_torch(wl, device="cuda")
    names = ("q", "k", "v", "alpha", "b", "w")
    o, S_T = g.chunk_fwd(*[ins[n] for n in names], ins["S0"])
    torch.cuda.synchronize()
    heads = [0, 11]
    sub = {n: ins[n][:, :, heads].cpu() for n in names}
    o_ref, S_ref = oracle.forward(*[sub[n] for n in names], ins["S0"][:, heads].cpu())
    for i, h in enumerate(heads):
        eo = normwise_err(o[:, :, h:h + 1], o_ref[:, :, i:i + 1])
        es = normwise_err(S_T[:, h:h + 1], S_ref[:, i:i + 1])
        print(f"  head {h}: o err {eo:.2e}  S_T err {es:.2e}", flush=True)
        assert eo <= TOL16 and es <= TOL16, (h, eo, es)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_chunk_sequence_beyond_4gib(schedule):
    """One sequence of T = 600,000 tokens at H16 d128: its o rows span 4.9 GB, past the 4 GiB a
    32-bit byte offset reaches (rows from token 524,288 on). The first P = 520,000 tokens of every
    head carry alpha = 1, b = w = 0 (the state stays S0, so o_t = S0^T q_t, checked in closed
    form); the last 80,000 tokens carry the workload's gates and are checked against the oracle
    started from S0. Two sampled heads."""
    from gated_delta_rule_25_amd.inputs import make_inputs_torch
    T, P = 600_000, 520_000
    banner(f"chunk T={T} (o past 4 GiB), schedule {schedule}, heads 3 and 14")
    g = _g()
    wl = scaled(WORKLOADS["long_prefill"], T=T, seed=20261)
    ins = make_inputs_torch(wl, device="cuda")
    ins["alpha"][:, :P] = 1.0
    ins["b"][:, :P] = 0.0
    ins["w"][:, :P] = 0.0
    names = ("q", "k", "v", "alpha", "b", "w")
    o, S_T = g.chunk_fwd(*[ins[n] for n in names], ins["S0"], schedule=schedule)
    torch.cuda.synchronize()
    heads = [3, 14]
    S0 = ins["S0"][:, heads].double().cpu().numpy()
    sub = {n: ins[n][:, P:, heads].cpu() for n in names}
    o_tail, S_ref = oracle.forward(*[sub[n] for n in names], S0)
    for i, h in enumerate(heads):
        q_pre = ins["q"][0, :P, h].double().cpu().numpy()
        o_pre = q_pre @ S0[0, i]  # o_t = S0^T q_t while the state stays S0
        e_pre = normwise_err(o[0, :P, h], o_pre)
        e_tail = normwise_err(o[:, P:, h:h + 1], o_tail[:, :, i:i + 1])
        es = normwise_err(S_T[:, h:h + 1], S_ref[:, i:i + 1])
        print(f"  head {h}: o[:P] {e_pre:.2e}  o[P:] {e_tail:.2e}  S_T {es:.2e}", flush=True)
        assert e_pre <= TOL16 and e_tail <= TOL16 and es <= TOL16, (h, e_pre, e_tail, es)


D256_CASES = [
    ("bf16_d256_ragged", scaled(WORKLOADS["prefill_1p3b"], B=2, T=200, H=2, d_k=256, d_v=256)),
    ("bf16_d256_T1", scaled(WORKLOADS["prefill_1p3b"], B=1, T=1, H=2, d_k=256, d_v=256)),
    ("bf16_d256_T65", scaled(WORKLOADS["prefill_1p3b"], B=1, T=65, H=3, d_k=256, d_v=256)),
    ("bf16_d256_gdn", scaled(WORKLOADS["gdn_scalar"], B=1, T=257, H=2, d_k=256, d_v=256)),
    ("bf16_d256_kda", scaled(WORKLOADS["kda_scalar"], B=2, T=130, H=2, d_k=256, d_v=256)),
    ("bf16_d256_strong_decay", scaled(WORKLOADS["prefill_1p3b"], B=1, T=190, H=2, d_k=256, d_v=256,
                                      alpha_mu=-2.0)),
    # one sequence of 47 chunks on 2 heads: few enough workgroups that the sequence is cut into
    # segments (the state-only transition pass, the scan, then all segments at once)
    ("bf16_d256_segmented", scaled(WORKLOADS["long_prefill"], B=1, T=3000, H=2, d_k=256, d_v=256)),
]


@pytest.mark.parametrize("name,wl", D256_CASES, ids=[c[0] for c in D256_CASES])
def test_chunk_d256_matches_oracle(name, wl):
    """Head size 256 on the two-kernel path (bf16, with a workspace: one block buffer in the
    chain kernel); the page "NVIDIA улучшила память LLM…", section "Аналитика", sizes the state by
    its total, which a 256 x 256 head also meets."""
    banner(f"chunk d256 {name} {wl}")
    _check(name, make_inputs(wl), TOL16, "split")


def test_chunk_d256_needs_a_workspace():
    g = _g()
    ins = _cuda(make_inputs(scaled(WORKLOADS["prefill_1p3b"], B=1, T=64, H=1, d_k=256, d_v=256)))
    with pytest.raises(g.Gdn2Error):
        g.chunk_fwd(ins["q"], ins["k"], ins["v"], ins["alpha"], ins["b"], ins["w"], ins["S0"], schedule="fused")
