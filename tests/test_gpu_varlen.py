"""GPU parity: the packed (ragged) prefill gdn2_chunk_fwd_varlen against the fp64 oracle, run
sequence by sequence.

Every sequence of the packed batch is its own recurrence from its own initial state, so the
oracle runs each one alone ([1, L, H, d] slices of the packed rows) and the packed o and S_T
are compared with its results. Bars as for the two-kernel prefill: 2e-3 (bf16 inputs), 1e-5
(fp32 inputs). Length mixes cover empty sequences, one token, chunk-1, one chunk, chunk+1 and
several chunks with a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import banner, normwise_err
from gated_delta_rule_25_amd.inputs import WORKLOADS, make_packed_inputs, packed_lengths, scaled

pytestmark = pytest.mark.gpu

TOL16, TOL32 = 2e-3, 1e-5
NAMES = ("q", "k", "v", "alpha", "b", "w")


def _g():
    import gated_delta_rule_25_amd as g
    return g


def _oracle_seq(ins, lo, hi, s, prologue=None):
    """The oracle on rows lo..hi-1 as one sequence from initial state s."""
    x = {n: (None if ins[n] is None else ins[n][lo:hi].unsqueeze(0)) for n in NAMES}
    S0 = None if ins["S0"] is None else ins["S0"][s:s + 1]
    q, k, a, b, w = x["q"], x["k"], x["alpha"], x["b"], x["w"]
    if prologue is not None:
        q, k, a, b, w = oracle.prologue(q, k, a, b, w, l2norm=prologue[0], gate_logits=prologue[1])
    if ins["alpha_scalar"] or ins["beta_scalar"]:
        a, b, w = oracle.broadcast_gates(a, b, w, q.shape[-1], x["v"].shape[-1],
                                         alpha_scalar=ins["alpha_scalar"], beta_scalar=ins["beta_scalar"])
    o, S = oracle.forward(q, k, x["v"], a, b, w, S0)
    return np.asarray(o)[0], np.asarray(S)[0]


def _run(ins, **kw):
    d = {n: (None if ins[n] is None else ins[n].cuda()) for n in NAMES}
    S0 = None if ins["S0"] is None else ins["S0"].cuda()
    o, S = _g().chunk_fwd_varlen(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], ins["cu_seqlens"].cuda(),
                                 S0, **kw)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def _check(ins, o, S, tol, bounds=None, prologue=None, seqs=None):
    cu = ins["cu_seqlens"].tolist() if bounds is None else bounds
    N = len(cu) - 1
    worst = 0.0
    for s in (range(N) if seqs is None else seqs):
        lo, hi = cu[s], cu[s + 1]
        if hi == lo:  # no tokens: the state passes through unchanged
            ref = np.zeros_like(S[s].numpy()) if ins["S0"] is None else ins["S0"][s].numpy()
            assert np.array_equal(S[s].numpy(), ref), s
            continue
        o_ref, S_ref = _oracle_seq(ins, lo, hi, s, prologue)
        eo, es = normwise_err(o[lo:hi], o_ref), normwise_err(S[s], S_ref)
        worst = max(worst, eo, es)
        assert eo <= tol and es <= tol, (s, lo, hi, eo, es)
    print(f"  worst err {worst:.2e}", flush=True)


MIX = [0, 1, 63, 64, 65, 200, 0, 130, 17, 257]
CASES = [
    ("bf16_d128_general", scaled(WORKLOADS["prefill_1p3b"], H=2), MIX, TOL16),
    ("bf16_d64_general", scaled(WORKLOADS["prefill_1p3b"], H=3, d_k=64, d_v=64), [5, 0, 128, 300], TOL16),
    ("bf16_d32_general", scaled(WORKLOADS["prefill_1p3b"], H=2, d_k=32, d_v=32), [70, 1, 190], TOL16),
    ("bf16_gdn", scaled(WORKLOADS["gdn_scalar"], H=2), [100, 64, 3], TOL16),
    ("bf16_kda", scaled(WORKLOADS["kda_scalar"], H=2), [3, 150, 0], TOL16),
    ("bf16_zero_S0", scaled(WORKLOADS["prefill_1p3b"], H=2, s0_std=0.0), [90, 40], TOL16),
    ("fp32_d32", scaled(WORKLOADS["tiny_fp32"], s0_std=0.1), [0, 77, 64, 129], TOL32),
    ("fp32_d64", scaled(WORKLOADS["prefill_1p3b"], H=2, d_k=64, d_v=64, dtype="fp32"), [5, 130, 1, 64], TOL32),
    ("fp32_d128", scaled(WORKLOADS["prefill_1p3b"], H=2, dtype="fp32"), [0, 77, 200, 65], TOL32),
    ("fp32_d128_kda", scaled(WORKLOADS["kda_scalar"], H=2, dtype="fp32"), [90, 3], TOL32),
]


@pytest.mark.parametrize("name,wl,lengths,tol", CASES, ids=[c[0] for c in CASES])
def test_varlen_matches_oracle_per_sequence(name, wl, lengths, tol):
    banner(f"varlen {name} lengths={lengths} {wl}")
    ins = make_packed_inputs(wl, lengths)
    o, S = _run(ins)
    _check(ins, o, S, tol)


@pytest.mark.parametrize("l2n,gl", [(True, True), (False, True)])
def test_varlen_prologue(l2n, gl):
    wl = scaled(WORKLOADS["prefill_1p3b"], H=2)
    banner(f"varlen prologue l2norm={l2n} logits={gl}")
    ins = make_packed_inputs(wl, [70, 0, 129, 5], raw=True)
    if not l2n:  # the kernel normalises nothing: hand it unit keys and queries
        q, k, _, _, _ = oracle.prologue(ins["q"], ins["k"], ins["alpha"], ins["b"], ins["w"],
                                        l2norm=True, gate_logits=False)
        ins["q"], ins["k"] = (torch.from_numpy(np.asarray(x)).to(torch.bfloat16) for x in (q, k))
    o, S = _run(ins, l2norm=l2n, gate_logits=gl)
    _check(ins, o, S, TOL16, prologue=(l2n, gl))


def test_varlen_equal_lengths_equal_the_batched_call():
    # N sequences of one length packed: the same kernels on the same blocks as chunk_fwd with
    # B = N, so the two results agree to the last bit
    wl = scaled(WORKLOADS["prefill_1p3b"], H=3)
    N, L = 4, 200
    banner(f"varlen vs batched, N={N} L={L}")
    ins = make_packed_inputs(wl, [L] * N)
    o, S = _run(ins)
    d = {n: ins[n].reshape(N, L, *ins[n].shape[1:]).cuda() for n in NAMES}
    o2, S2 = _g().chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], ins["S0"].cuda())
    torch.cuda.synchronize()
    assert torch.equal(o, o2.cpu().reshape(N * L, *o2.shape[2:]))
    assert torch.equal(S, S2.cpu())


def test_varlen_all_sequences_empty():
    wl = scaled(WORKLOADS["prefill_1p3b"], H=2)
    banner("varlen, every sequence empty")
    ins = make_packed_inputs(wl, [0, 0, 0])
    o, S = _run(ins)
    assert o.shape[0] == 0
    assert torch.equal(S, ins["S0"])


def test_varlen_bounds_are_clamped_into_the_batch():
    # cu = [3, 100, 50, 250, 180] over 200 rows: clamped to [0, 200] and made non-decreasing,
    # the sequences are rows 3..99, (empty), 100..199, (empty); rows 0..2 belong to none and
    # keep what o held
    wl = scaled(WORKLOADS["prefill_1p3b"], H=2)
    banner("varlen, bounds out of order and past the end")
    ins = make_packed_inputs(wl, [200, 0, 0, 0])
    ins["cu_seqlens"] = torch.tensor([3, 100, 50, 250, 180], dtype=torch.int32)
    o_buf = torch.full((200, 2, 128), 7.0, device="cuda")
    o, S = _run(ins, o=o_buf)
    assert torch.all(o[:3] == 7.0)
    _check(ins, o, S, TOL16, bounds=[3, 100, 100, 200, 200])


def test_varlen_full_size_sampled():
    # 32 sequences in a length mix, 32,768 rows in all, 16 heads of 128 x 128: the packed
    # counterpart of the B8 T4096 prefill; three sequences checked against the oracle
    wl = WORKLOADS["prefill_1p3b"]
    lengths = packed_lengths(32, 32768, seed=wl.seed)
    banner(f"varlen full size, 32 sequences, 32768 rows, H16 d128")
    ins = make_packed_inputs(wl, lengths)
    o, S = _run(ins)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    order = np.argsort(lengths)
    _check(ins, o, S, TOL16, seqs=[int(order[0]), int(order[len(order) // 2]), int(order[-1])])


def test_varlen_many_sequences_span_several_table_tiles():
    # 700 sequences (the sequence table is built in tiles of 256 bounds, carrying the running
    # maximum and chunk count from tile to tile), lengths 0..70 with many empty ones
    rng = np.random.default_rng(97)
    lengths = [int(x) for x in rng.integers(0, 71, 700)]
    lengths[255] = lengths[256] = lengths[511] = 0
    lengths[257] = 129
    wl = scaled(WORKLOADS["prefill_1p3b"], H=1, d_k=32, d_v=32)
    banner(f"varlen, {len(lengths)} sequences, {sum(lengths)} rows, H1 d32")
    ins = make_packed_inputs(wl, lengths)
    o, S = _run(ins)
    _check(ins, o, S, TOL16)


def test_varlen_sequences_past_the_top_length_bucket():
    # the chains take the sequences longest first, ordered by chunk count in 1024 buckets; two
    # sequences of more than 1023 chunks share the top bucket (H1 d32, 136,075 rows)
    wl = scaled(WORKLOADS["prefill_1p3b"], H=1, d_k=32, d_v=32)
    lengths = [70000, 5, 0, 66000, 70]
    banner(f"varlen, lengths {lengths}, H1 d32")
    ins = make_packed_inputs(wl, lengths)
    o, S = _run(ins)
    _check(ins, o, S, TOL16)
