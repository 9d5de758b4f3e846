"""GPU parity for the serving shapes: decode over a pool of states (slot-indexed) and head size 256
on the decode and token-by-token paths, against the fp64 oracle (bar 1e-5: fp32 arithmetic)."""
import numpy as np
import pytest
import torch

import oracle
from parity import banner, normwise_err
from gated_delta_rule_25_amd.inputs import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu
TOL32 = 1e-5


def _g():
    import gated_delta_rule_25_amd as g
    return g


def test_decode_slots_matches_oracle_and_skips_padding():
    banner("decode over a state pool: B 5 rows, 9 slots, one padding row")
    wl = scaled(WORKLOADS["prefill_1p3b"], B=5, T=1, H=3)
    ins = make_inputs(wl)
    rng = np.random.default_rng(41)
    n_slots = 9
    pool = torch.from_numpy(rng.standard_normal((n_slots, 3, 128, 128)).astype(np.float32) * 0.1)
    slots = torch.tensor([7, 2, -1, 0, 8], dtype=torch.int32)
    d = {n: ins[n][:, 0].cuda() for n in ("q", "k", "v", "alpha", "b", "w")}
    gpool = pool.cuda()
    o = torch.full((5, 3, 128), 123.0, device="cuda")
    _g().decode_step_slots(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], gpool, slots.cuda(), o=o)
    torch.cuda.synchronize()
    live = [0, 1, 3, 4]
    S = pool[slots[live].long()]
    o_ref, S_ref = oracle.decode_step(*(ins[n][live, 0] for n in ("q", "k", "v", "alpha", "b", "w")), S)
    eo = normwise_err(o[live], o_ref)
    es = normwise_err(gpool[slots[live].long()], S_ref)
    print(f"  o err {eo:.2e}  S err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32
    assert torch.all(o[2] == 123.0)  # the padding row is skipped
    untouched = [i for i in range(n_slots) if i not in (7, 2, 0, 8)]
    assert torch.equal(gpool[untouched].cpu(), pool[untouched])


@pytest.mark.parametrize("path", ["decode", "recurrent"])
def test_head_size_256(path):
    T = 1 if path == "decode" else 40
    wl = scaled(WORKLOADS["prefill_1p3b"], B=2, T=T, H=2, d_k=256, d_v=256)
    banner(f"head size 256, {path} {wl}")
    ins = make_inputs(wl)
    o_ref, S_ref = oracle.forward(*(ins[n] for n in ("q", "k", "v", "alpha", "b", "w")), ins["S0"])
    d = {n: ins[n].cuda() for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    g = _g()
    if path == "decode":
        S = d["S0"].clone()
        o = g.decode_step(*(d[n][:, 0] for n in ("q", "k", "v", "alpha", "b", "w")), S)
        o_ref = o_ref[:, 0]
    else:
        o, S = g.recurrent_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], d["S0"])
    torch.cuda.synchronize()
    eo, es = normwise_err(o, o_ref), normwise_err(S, S_ref)
    print(f"  {path}: o err {eo:.2e}  S err {es:.2e}", flush=True)
    assert eo <= TOL32 and es <= TOL32
