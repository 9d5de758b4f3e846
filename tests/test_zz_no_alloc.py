"""GPU test of the allocation-free entry point gdn2_rmsnorm_bwd_noalloc (through the C ABI): its
outputs equal those of gdn2_rmsnorm_bwd (same kernels, the dweight partials in the library's fixed
device scratch instead of a caller workspace) bit for bit, over calls in a row whose sizes shrink,
so that partials a larger earlier call left in the scratch are never read. Also checked against
the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import banner, normwise_err

pytestmark = pytest.mark.gpu


def _inputs(rows, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    scale = np.exp(rng.uniform(np.log(1e-2), np.log(1e2), (rows, 1)))
    x = (rng.standard_normal((rows, d)) * scale).astype(np.float32)
    w = rng.standard_normal(d).astype(np.float32)
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    return x, w, dy


def test_rmsnorm_bwd_noalloc_equals_workspace_entry_point():
    import gated_delta_rule_25_amd as g
    # largest first (1024 partials), then smaller ones: a later call must not read the earlier
    # call's partials left in the shared scratch
    for rows, d, eps, weighted in ((100_003, 128, 1e-6, True), (4099, 256, 0.0, True), (37, 64, 0.1, False),
                                   (1, 32, 1e-6, True), (0, 128, 1e-6, True)):
        banner(f"rmsnorm_bwd_noalloc rows={rows} d={d} eps={eps} weight={weighted}")
        x, w, dy = _inputs(rows, d, seed=7 * rows + d)
        xc, dyc = torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda()
        wc = torch.from_numpy(w).cuda() if weighted else None
        ref = g.rmsnorm_bwd(xc, wc, dyc, eps=eps)
        dx = torch.empty_like(xc)
        dw = torch.full((d,), float("nan"), device="cuda")
        got = g.rmsnorm_bwd_noalloc(xc, wc, dyc, eps=eps, dx=dx, dweight=dw)
        torch.cuda.synchronize()
        assert got["dx"].data_ptr() == dx.data_ptr() and got["dweight"].data_ptr() == dw.data_ptr()
        assert torch.equal(dx, ref["dx"]), "dx differs from gdn2_rmsnorm_bwd"
        assert torch.equal(dw, ref["dweight"]), "dweight differs from gdn2_rmsnorm_bwd"
        if rows == 0:
            assert torch.equal(dw, torch.zeros_like(dw))
            continue
        rb = oracle.rmsnorm_backward(x, w if weighted else None, dy, eps=eps)
        e_dx, e_dw = normwise_err(dx.cpu(), rb["dx"]), normwise_err(dw.cpu(), rb["dweight"])
        print(f"  dx {e_dx:.2e}  dweight {e_dw:.2e}", flush=True)
        assert e_dx <= 1e-5 and e_dw <= 1e-5, (e_dx, e_dw)
    # without dweight the scratch is not touched, dx alone
    x, w, dy = _inputs(50, 128, seed=11)
    xc, dyc, wc = torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda(), torch.from_numpy(w).cuda()
    dx = torch.empty_like(xc)
    g.rmsnorm_bwd_noalloc(xc, wc, dyc, eps=1e-6, dx=dx, dweight=None)
    ref = g.rmsnorm_bwd(xc, wc, dyc, eps=1e-6, need_dweight=False)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref["dx"])
