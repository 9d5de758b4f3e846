"""GPU parity of the sparse delta memory (gdn2_sdm_address, gdn2_sdm_fwd, gdn2_sdm_fold) against
the fp64 oracle (``oracle/sdm.py``), through the C ABI.

Memory update: the kernels run in fp32 (decay sums in fp64) on inputs the oracle sees exactly
(bf16 or fp32 values upcast), so o and the memory (each slot's stored row times exp(L - stamp))
are held to 1e-5 normwise, the bar of the other fp32-state
paths. Addressing: the kernel scores in fp32 and the oracle in fp64, so where two pair sums lie
within rounding of each other at the edge of the top m, either choice is correct. Each query's
chosen slots are compared with the oracle's; where they differ, the chosen set must be a valid top
m: its fp64 sums, sorted, equal the oracle's within 2e-5. Weights are checked against the softmax
of the fp64 sums of the slots the kernel chose.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_25_amd.inputs import make_sdm_inputs
from parity import banner, normwise_err, to64

pytestmark = pytest.mark.gpu

TOL = 1e-5
SCORE_TOL = 2e-5
MARGIN = 3e-5


def memory_now(state):
    """The memory a state (M, stamp, L) stands for: M[s] * exp(L - stamp[s]) per column tile
    (float64, on the host)."""
    M, stamp, L = (x.detach().double().cpu().numpy() for x in state)  # stamps and L stay fp64
    B, H, N, dv = M.shape
    tiles = dv // 64
    f = np.exp(L[:, :, :, None] - stamp)                       # [B, H, tiles, N]
    return (M.reshape(B, H, N, tiles, 64) * f.transpose(0, 1, 3, 2)[..., None]).reshape(B, H, N, dv)


def _run_fwd(g, d, B, T, H, N, dv, W, R, *, with_w=True, widx=None, ridx=None, wwt=None, rwt=None, M0=None):
    dev = "cuda"
    widx = d["widx"] if widx is None else widx
    ridx = d["ridx"] if ridx is None else ridx
    wwt = d["wwt"] if wwt is None else wwt
    rwt = d["rwt"] if rwt is None else rwt
    M0 = d["M0"] if M0 is None else M0
    state = g.sdm_state(M0.to(dev).clone())
    o = g.sdm_fwd(d["v"].to(dev), d["alpha"].to(dev), d["b"].to(dev), d["w"].to(dev) if with_w else None,
                  widx.to(dev), wwt.to(dev), ridx.to(dev), rwt.to(dev), state)
    torch.cuda.synchronize()
    return o, state


def _oracle_fwd(d, *, with_w=True, widx=None, ridx=None, wwt=None, rwt=None, M0=None):
    pick = lambda x, dflt: to64(dflt if x is None else x)  # noqa: E731
    return oracle.sdm_forward(to64(d["v"]), to64(d["alpha"]), to64(d["b"]), to64(d["w"]) if with_w else None,
                              pick(widx, d["widx"]).astype(np.int64), pick(wwt, d["wwt"]),
                              pick(ridx, d["ridx"]).astype(np.int64), pick(rwt, d["rwt"]), pick(M0, d["M0"]))


CASES = {
    # name: (B, T, H, n, dv, W, R, dtype, alpha_mu)
    "bf16_dv64_N1024": (2, 100, 3, 32, 64, 64, 64, "bf16", 3.0),
    "fp32_dv128_W16_R8": (1, 64, 2, 64, 128, 16, 8, "fp32", 3.0),
    "bf16_dv256_N256_overlaps": (1, 40, 2, 16, 256, 64, 64, "bf16", 3.0),
    "strong_decay_folds": (1, 300, 2, 32, 128, 32, 32, "bf16", -1.0),
    "decode_T1": (4, 1, 3, 64, 128, 64, 64, "bf16", 3.0),
    # list lengths that split unevenly over the four wavefronts' 16-position parts, in a memory
    # of 64 slots, so nearly every read slot is also written and every token rewrites the last
    "bf16_dv64_W37_R50_N64": (2, 60, 2, 8, 64, 37, 50, "bf16", 3.0),
    "fp32_dv128_W1_R1": (1, 50, 2, 16, 128, 1, 1, "fp32", 3.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_sdm_fwd_matches_oracle(name):
    import gated_delta_rule_25_amd as g
    B, T, H, n, dv, W, R, dt, amu = CASES[name]
    banner(f"sdm_fwd {name}")
    d = make_sdm_inputs(B, T, H, 64, dv, n, W, R, seed=31 + len(name), dtype=dt, alpha_mu=amu)
    o, state = _run_fwd(g, d, B, T, H, d["N"], dv, W, R)
    o_ref, M_ref = _oracle_fwd(d)
    eo, em = normwise_err(o, o_ref), normwise_err(memory_now(state), M_ref)
    print(f"  o {eo:.2e}  memory {em:.2e}  L in [{state[2].min().item():.4g}, {state[2].max().item():.4g}]",
          flush=True)
    assert eo <= TOL and em <= TOL, (eo, em)


def test_sdm_fwd_without_write_gate_and_reads_of_written_slots():
    """w = None (ones), and every token reads exactly the slots it writes (the read must see the
    token's own writes)."""
    import gated_delta_rule_25_amd as g
    B, T, H, n, dv, W = 1, 50, 2, 32, 128, 48
    banner("sdm_fwd w=None, read slots = write slots")
    d = make_sdm_inputs(B, T, H, 64, dv, n, W, W, seed=77)
    o, state = _run_fwd(g, d, B, T, H, d["N"], dv, W, W, with_w=False, ridx=d["widx"], rwt=d["wwt"])
    o_ref, M_ref = _oracle_fwd(d, with_w=False, ridx=d["widx"], rwt=d["wwt"])
    eo, em = normwise_err(o, o_ref), normwise_err(memory_now(state), M_ref)
    print(f"  o {eo:.2e}  memory {em:.2e}", flush=True)
    assert eo <= TOL and em <= TOL


def test_sdm_fwd_skips_slots_outside_the_memory():
    """A write or read slot outside [0, N) is skipped, as if its weight were 0."""
    import gated_delta_rule_25_amd as g
    B, T, H, n, dv, W = 1, 20, 1, 16, 64, 8
    banner("sdm_fwd out-of-range slots")
    d = make_sdm_inputs(B, T, H, 64, dv, n, W, W, seed=5)
    N = d["N"]
    widx, ridx = d["widx"].clone(), d["ridx"].clone()
    widx[..., 0] = N + 7
    ridx[..., 1] = -3
    o, state = _run_fwd(g, d, B, T, H, N, dv, W, W, widx=widx, ridx=ridx)
    # the oracle takes distinct in-range slots: an unused slot at weight 0 stands for the skip
    wo, ro = d["widx"].numpy().copy(), d["ridx"].numpy().copy()
    ww, rw = d["wwt"].numpy().astype(np.float64), d["rwt"].numpy().astype(np.float64)
    for t in range(T):
        free_w = np.setdiff1d(np.arange(N), wo[0, t, 0])[0]
        wo[0, t, 0, 0], ww[0, t, 0, 0] = free_w, 0.0
        ro[0, t, 0, 1], rw[0, t, 0, 1] = 0, 0.0
    o_ref, M_ref = _oracle_fwd(d, widx=wo, wwt=ww, ridx=ro, rwt=rw)
    eo, em = normwise_err(o, o_ref), normwise_err(memory_now(state), M_ref)
    assert eo <= TOL and em <= TOL, (eo, em)


def test_sdm_fwd_split_equals_one_call_and_fold():
    """Two calls (T1 then T2 tokens) leave the same memory, stamps, L and outputs as one call of
    T1 + T2 tokens, bit for bit; gdn2_sdm_fold then gives the memory itself with every stamp = L.
    Includes alpha = 0 tokens (the memory is wiped)."""
    import gated_delta_rule_25_amd as g
    B, T, H, n, dv, W = 2, 90, 2, 32, 128, 64
    banner("sdm_fwd split + fold")
    d = make_sdm_inputs(B, T, H, 64, dv, n, W, W, seed=9, alpha_mu=0.0)
    d["alpha"][:, 50] = 0.0
    dev = "cuda"
    keys = ("v", "alpha", "b", "w", "widx", "wwt", "ridx", "rwt")
    args = {k: d[k].to(dev) for k in keys}
    s1 = g.sdm_state(d["M0"].to(dev).clone())
    o1 = g.sdm_fwd(*(args[k] for k in keys), s1)
    s2 = g.sdm_state(d["M0"].to(dev).clone())
    parts = []
    for lo, hi in ((0, 37), (37, T)):
        sl = {k: v[:, lo:hi].contiguous() for k, v in args.items()}
        parts.append(g.sdm_fwd(*(sl[k] for k in keys), s2))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=1), o1)
    assert all(torch.equal(x, y) for x, y in zip(s1, s2))
    want = memory_now(s1)
    g.sdm_fold(s1)
    torch.cuda.synchronize()
    M, stamp, L = s1
    assert torch.equal(stamp, L[..., None].expand_as(stamp))
    assert np.allclose(to64(M), want, rtol=1e-6, atol=1e-30)
    o_ref, M_ref = _oracle_fwd(d)
    assert normwise_err(o1, o_ref) <= TOL and normwise_err(M, M_ref) <= TOL


def test_sdm_decode_full_size_sampled_heads():
    """One decode step at B = 8, H = 16, N = 65,536 slots of d_v = 128 (32 MiB per head), W = R = 64,
    checked against the oracle on four sampled heads."""
    import gated_delta_rule_25_amd as g
    B, H, n, dv, W = 8, 16, 256, 128, 64
    N = n * n
    banner("sdm decode B8 H16 N65536")
    d = make_sdm_inputs(B, 1, H, 128, dv, n, W, W, seed=404, with_memory=False)
    gen = torch.Generator(device="cuda").manual_seed(405)
    M = torch.randn(B, H, N, dv, device="cuda", generator=gen) * 0.1
    M0_heads = {}
    rng = np.random.Generator(np.random.PCG64(406))
    heads = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(4)]
    for bb, hh in heads:
        M0_heads[(bb, hh)] = M[bb, hh].double().cpu().numpy()
    dev = "cuda"
    state = g.sdm_state(M)
    o = g.sdm_fwd(d["v"].to(dev), d["alpha"].to(dev), d["b"].to(dev), d["w"].to(dev), d["widx"].to(dev),
                  d["wwt"].to(dev), d["ridx"].to(dev), d["rwt"].to(dev), state)
    g.sdm_fold(state)
    torch.cuda.synchronize()
    for bb, hh in heads:
        sl = lambda x: to64(x[bb:bb + 1, :, hh:hh + 1])  # noqa: E731
        o_ref, M_ref = oracle.sdm_forward(sl(d["v"]), sl(d["alpha"]), sl(d["b"]), sl(d["w"]),
                                          sl(d["widx"]).astype(np.int64), sl(d["wwt"]),
                                          sl(d["ridx"]).astype(np.int64), sl(d["rwt"]),
                                          M0_heads[(bb, hh)][None, None])
        got_M = M[bb, hh].double().cpu().numpy()
        eo, em = normwise_err(o[bb:bb + 1, :, hh:hh + 1], o_ref), normwise_err(got_M, M_ref[0, 0])
        print(f"  head ({bb}, {hh}): o {eo:.2e} memory {em:.2e}", flush=True)
        assert eo <= TOL and em <= TOL


def _pair_sums64(x, C1, C2, h):
    """fp64 scores of all n^2 slots of one query (slot i * n + j)."""
    x, C1, C2 = to64(x), to64(C1[h]), to64(C2[h])
    half = C1.shape[1]
    return ((C1 @ x[:half])[:, None] + (C2 @ x[half:])[None, :]).ravel()


ADDR_CASES = {
    # name: (rows, H, d_k, n, m, dtype)
    "bf16_dk128_n256_m64": (300, 4, 128, 256, 64, "bf16"),
    "fp32_dk64_n64_m16": (200, 2, 64, 64, 16, "fp32"),
    "bf16_dk256_n512_m64": (60, 2, 256, 512, 64, "bf16"),
    "bf16_dk128_n128_m1": (100, 3, 128, 128, 1, "bf16"),
    "bf16_dk128_n64_m64": (100, 2, 128, 64, 64, "bf16"),
}


@pytest.mark.parametrize("name", sorted(ADDR_CASES))
def test_sdm_address_matches_oracle(name):
    import gated_delta_rule_25_amd as g
    rows, H, dk, n, m, dt = ADDR_CASES[name]
    banner(f"sdm_address {name}")
    d = make_sdm_inputs(1, rows, H, dk, 64, n, 1, 1, seed=1000 + rows + n, dtype=dt, with_memory=False)
    x, C1, C2 = d["k"], d["C1"], d["C2"]
    idx, wt = g.sdm_address(x.cuda(), C1.cuda(), C2.cuda(), m)
    torch.cuda.synchronize()
    idx, wt = idx.cpu().numpy(), wt.cpu().numpy().astype(np.float64)
    differ = 0
    xs = to64(x)
    for t in range(rows):
        for h in range(H):
            s = _pair_sums64(xs[0, t, h], C1, C2, h)
            r_idx, _ = oracle.pkm_address(xs[0, t, h], to64(C1[h]), to64(C2[h]), m)
            got = idx[0, t, h]
            assert len(set(got.tolist())) == m and got.min() >= 0 and got.max() < n * n
            if not np.array_equal(got, r_idx):
                differ += 1
                assert np.allclose(np.sort(s[got]), np.sort(s[r_idx]), rtol=0, atol=SCORE_TOL), (t, h)
            e = np.exp(s[got] - s[got].max())
            assert np.allclose(wt[0, t, h], e / e.sum(), rtol=0, atol=TOL), (t, h)
    print(f"  queries whose slots differ from the oracle's (valid ties): {differ} of {rows * H}", flush=True)
    assert differ <= max(2, rows * H // 100)


def test_sdm_address_then_update_end_to_end():
    """Addresses from gdn2_sdm_address (k for writes, q for reads) feeding gdn2_sdm_fwd, against
    oracle.pkm_address + oracle.sdm_forward on the same inputs. The seeded inputs are checked to
    hold no near-tie at the edge of any selection (every gap above MARGIN, beyond the fp32 error
    of a 64-term score), so both sides must pick the same slots."""
    import gated_delta_rule_25_amd as g
    B, T, H, dk, dv, n, W, R = 1, 60, 2, 128, 128, 64, 64, 32
    banner("sdm address + update end to end")
    d = make_sdm_inputs(B, T, H, dk, dv, n, W, R, seed=2029)  # smallest margin 6e-5
    q64, k64 = to64(d["q"]), to64(d["k"])
    C1, C2 = to64(d["C1"]), to64(d["C2"])
    widx = np.empty((B, T, H, W), np.int64)
    wwt = np.empty((B, T, H, W))
    ridx = np.empty((B, T, H, R), np.int64)
    rwt = np.empty((B, T, H, R))
    for t in range(T):
        for h in range(H):
            for x, m, I, A in ((k64[0, t, h], W, widx, wwt), (q64[0, t, h], R, ridx, rwt)):
                s = _pair_sums64(x, C1, C2, h)
                srt = np.sort(s)[::-1]
                assert srt[m - 1] - srt[m] > MARGIN, "near-tie in the seeded inputs"
                for tab, xh in ((C1[h], x[:dk // 2]), (C2[h], x[dk // 2:])):
                    hs = np.sort(tab @ xh)[::-1]
                    assert m == n or hs[m - 1] - hs[m] > MARGIN, "near-tie in the seeded inputs"
                i_, a_ = oracle.pkm_address(x, C1[h], C2[h], m)
                I[0, t, h], A[0, t, h] = i_, a_
    o_ref, M_ref = oracle.sdm_forward(to64(d["v"]), to64(d["alpha"]), to64(d["b"]), to64(d["w"]),
                                      widx, wwt, ridx, rwt, to64(d["M0"]))
    dev = "cuda"
    gw_idx, gw_wt = g.sdm_address(d["k"].to(dev), d["C1"].to(dev), d["C2"].to(dev), W)
    gr_idx, gr_wt = g.sdm_address(d["q"].to(dev), d["C1"].to(dev), d["C2"].to(dev), R)
    state = g.sdm_state(d["M0"].to(dev).clone())
    o = g.sdm_fwd(d["v"].to(dev), d["alpha"].to(dev), d["b"].to(dev), d["w"].to(dev), gw_idx, gw_wt, gr_idx,
                  gr_wt, state)
    torch.cuda.synchronize()
    assert np.array_equal(gw_idx.cpu().numpy(), widx) and np.array_equal(gr_idx.cpu().numpy(), ridx)
    eo, em = normwise_err(o, o_ref), normwise_err(memory_now(state), M_ref)
    print(f"  o {eo:.2e}  memory {em:.2e}", flush=True)
    assert eo <= TOL and em <= TOL
