"""The C-ABI library loads, exports every declared entry point, and rejects bad arguments
on the host. No call here reaches a kernel launch, so these run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")
LIB = os.path.join(ROOT, "gated_delta_rule_25_amd", "libgdn2.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libgdn2.so not built (run python -m gated_delta_rule_25_amd.build)")
    import gated_delta_rule_25_amd as g
    return g.load()


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ("gdn2_chunk_fwd", "gdn2_decode_step", "gdn2_recurrent_fwd",
                 "gdn2_chunk_fwd_workspace_bytes", "gdn2_status_str", "gdn2_abi_version"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in gdn2.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.gdn2_abi_version() == 1
    for code in range(9):
        assert lib.gdn2_status_str(code)
    assert lib.gdn2_status_str(8) == b"size beyond the library's fixed scratch"
    assert lib.gdn2_status_str(0) == b"ok"


P = ctypes.c_void_p
FAKE = [P(0x10000 * (i + 1)) for i in range(12)]  # distinct, 16-byte aligned, never dereferenced


def chunk_call(lib, ptrs=None, B=1, T=4, H=1, dk=32, dv=32, dt=0, flags=0, ws=None, wsb=0):
    p = list(FAKE[:9]) if ptrs is None else ptrs
    return lib.gdn2_chunk_fwd(*p, B, T, H, dk, dv, dt, flags, ws, wsb, None)


def test_chunk_rejects_bad_arguments(lib):
    assert chunk_call(lib, B=0) == 2
    assert chunk_call(lib, T=-1) == 2
    assert chunk_call(lib, dk=48) == 3
    assert chunk_call(lib, dv=256) == 3
    assert chunk_call(lib, dt=7) == 3
    assert chunk_call(lib, flags=4) == 3
    p = list(FAKE[:9])
    p[0] = None
    assert chunk_call(lib, p) == 1  # q missing
    p = list(FAKE[:9])
    p[7] = None
    assert chunk_call(lib, p) == 1  # o missing
    p = list(FAKE[:9])
    p[1] = P(0x20008)
    assert chunk_call(lib, p) == 4  # misaligned k
    p = list(FAKE[:9])
    p[7] = p[0]
    assert chunk_call(lib, p) == 5  # o overlaps q
    p = list(FAKE[:9])
    assert chunk_call(lib, p, flags=2) == 3  # beta scalar but w given


def test_long_sequences_take_the_forward_not_the_backward(lib):
    # One sequence whose o spans more than 4 GiB (600,000 x 16 x 128 x 4 B = 4.9 GB): the forward
    # kernels address each chunk's rows from a 64-bit base, so the two-kernel path sizes a
    # workspace for it (a slot per chunk plus the segment buffers); the backward still addresses
    # a sequence's rows with 32-bit offsets and refuses it.
    T = 600_000
    nch = (T + 63) // 64
    state = 16 * 128 * 128 * 4
    per_chunk = lib.gdn2_chunk_fwd_workspace_bytes(1, 64, 16, 128, 128, 0, 0) - state
    assert lib.gdn2_chunk_fwd_workspace_bytes(1, T, 16, 128, 128, 0, 0) >= state + nch * per_chunk
    assert lib.gdn2_chunk_bwd_workspace_bytes(1, T, 16, 128, 128, 0, 0) == 0
    far = [P(0x200000000 * (i + 1)) for i in range(16)]
    assert lib.gdn2_chunk_bwd(*far[:16], 1, T, 16, 128, 128, 0, 0, P(0x200000000 * 20), 1 << 40, None) == 3


def test_workspace_query_is_state_plus_one_slot_per_chunk(lib):
    q = lib.gdn2_chunk_fwd_workspace_bytes
    state = 8 * 16 * 128 * 128 * 4
    one = q(8, 64, 16, 128, 128, 0, 0)
    per_chunk = one - state
    assert per_chunk > 0 and per_chunk % 256 == 0
    assert q(8, 4096, 16, 128, 128, 0, 0) == state + 64 * per_chunk
    assert q(8, 4097, 16, 128, 128, 0, 0) == state + 65 * per_chunk  # ragged last chunk
    # fp32 at d = 128: the two-kernel path with fp32 operand blocks, larger than the bf16 ones
    per_chunk32 = q(8, 64, 16, 128, 128, 1, 0) - state
    assert per_chunk32 > per_chunk and per_chunk32 % 256 == 0
    assert q(8, 4096, 16, 128, 128, 1, 0) == state + 64 * per_chunk32
    assert q(8, 4096, 16, 256, 256, 1, 0) == 0  # fp32 at d = 256: no two-kernel path


def test_chunk_rejects_partial_state_alias(lib):
    p = list(FAKE[:9])
    p[6] = P(0x900000)
    p[8] = P(0x900010)  # S_out overlaps S0 without being equal
    assert chunk_call(lib, p) == 5


def test_decode_rejects_bad_arguments(lib):
    f = lib.gdn2_decode_step
    p = list(FAKE[:8])
    assert f(*p, 0, 1, 128, 128, 0, 0, None) == 2
    assert f(*p, 1, 1, 96, 128, 0, 0, None) == 3
    q = list(p)
    q[6] = None  # S missing
    assert f(*q, 1, 1, 128, 128, 0, 0, None) == 1
    q = list(p)
    q[7] = q[6]  # o overlaps S
    assert f(*q, 1, 1, 128, 128, 0, 0, None) == 5


def test_recurrent_rejects_bad_arguments(lib):
    f = lib.gdn2_recurrent_fwd
    p = list(FAKE[:9])
    assert f(*p, 1, 4, 0, 64, 64, 0, 0, None) == 2
    assert f(*p, 1, 4, 1, 64, 16, 0, 0, None) == 3


def test_decode_slots_rejects_bad_arguments(lib):
    f = lib.gdn2_decode_step_slots
    p = list(FAKE[:6])
    pool, slots, o = FAKE[6], FAKE[7], FAKE[8]
    assert f(*p, pool, slots, o, 2, 1, 128, 128, 0, 0, 0, None) == 2      # no slots in the pool
    assert f(*p, pool, None, o, 2, 1, 128, 128, 4, 0, 0, None) == 1       # slots missing
    assert f(*p, None, slots, o, 2, 1, 128, 128, 4, 0, 0, None) == 1      # pool missing
    assert f(*p, pool, P(0x80002), o, 2, 1, 128, 128, 4, 0, 0, None) == 4  # slots misaligned
    assert f(*p, pool, slots, o, 2, 1, 96, 128, 4, 0, 0, None) == 3       # head size
    assert f(*p, pool, slots, o, 2, 1, 128, 128, 4, 0, 16, None) == 3     # unknown flag
    # the pool overlapping an input
    assert f(*p, P(0x10000), slots, o, 2, 1, 128, 128, 4, 0, 0, None) == 5


def test_head_size_256_on_the_chunked_prefill(lib):
    # d = 256 is taken by the two-kernel path only: bf16 with a workspace. Without a workspace,
    # with fp32, or in packed batches and the backward, it is refused on the host (no launch).
    far = [P(0x200000000 * (i + 1)) for i in range(9)]  # 8 GiB apart: nothing overlaps
    assert chunk_call(lib, far, dk=256, dv=256) == 3                  # no workspace
    assert chunk_call(lib, far, dk=256, dv=256, dt=1, ws=P(0x200000000 * 20), wsb=1 << 30) == 3  # fp32
    q = lib.gdn2_chunk_fwd_workspace_bytes
    state = 2 * 16 * 256 * 256 * 4
    one = q(2, 64, 16, 256, 256, 0, 0)
    assert one > state and (one - state) % 256 == 0
    # a slot per chunk (plus segment buffers: 2 x 16 heads x 4 tiles do not fill the chip)
    assert q(2, 4096, 16, 256, 256, 0, 0) >= state + 64 * (one - state)
    assert q(2, 4096, 16, 256, 256, 1, 0) == 0
    assert lib.gdn2_chunk_fwd_varlen_workspace_bytes(4, 4096, 16, 256, 256, 0, 0) == 0
    assert lib.gdn2_chunk_bwd_workspace_bytes(2, 4096, 16, 256, 256, 0, 0) == 0


def test_varlen_rejects_bad_arguments(lib):
    f = lib.gdn2_chunk_fwd_varlen
    qs = lib.gdn2_chunk_fwd_varlen_workspace_bytes
    p = [P(0x200000000 * (i + 1)) for i in range(9)]  # 8 GiB apart: nothing overlaps
    cu = P(0x200000000 * 10)
    ws = P(0x200000000 * 11)
    need = qs(4, 1000, 2, 128, 128, 0, 0)
    # table (4 N + 1 ints, padded to 256 B) then (T + 63 N) / 64 = 19 chunks per head
    assert need == 256 + 19 * 2 * (qs(1, 64, 1, 128, 128, 0, 0) - 256)
    assert qs(4, 1000, 2, 128, 128, 1, 0) > need    # fp32 at d = 128: larger operand blocks
    assert qs(4, 1000, 2, 256, 256, 0, 0) == 0      # head size 256: not in packed batches
    assert qs(0, 1000, 2, 128, 128, 0, 0) == 0

    def call(ptrs=p, cu=cu, N=4, T=1000, H=2, dk=128, dv=128, dt=0, flags=0, ws=ws, wsb=need):
        return f(*ptrs, cu, N, T, H, dk, dv, dt, flags, ws, wsb, None)

    assert call(N=0) == 2
    assert call(T=-1) == 2
    assert call(cu=None) == 1
    assert call(cu=P(0x200000000 * 10 + 2)) == 4
    assert call(ws=None) == 7
    assert call(wsb=need - 1) == 7
    assert call(ws=P(0x200000000 * 11 + 128)) == 4     # workspace not 256-byte aligned
    assert call(dk=256, dv=256) == 3
    assert call(dt=1) == 7                             # fp32 at d = 128: the bf16 workspace is too small
    assert call(flags=32) == 3
    assert call(cu=P(0x200000000 * 8)) == 5            # cu_seqlens overlaps o
    q = list(p)
    q[7] = q[1]
    assert call(ptrs=q) == 5                           # o overlaps k
    assert call(ws=P(0x200000000 * 7)) == 5            # workspace over S0


def test_chunked_calls_reject_grids_beyond_31_bits(lib):
    # B*H*chunks workgroups of 256 threads (four per chunk in the backward's key pass at d = 128)
    # past 2^31 threads: refused on the host. Pointers 1 TiB apart so nothing overlaps.
    far = [P((1 << 40) * (i + 1)) for i in range(16)]
    B, T, H = 32, 64 * 1024, 64
    assert lib.gdn2_chunk_fwd(*far[:9], B, T, H, 128, 128, 0, 0, None, 0, None) == 2
    assert lib.gdn2_chunk_bwd(*far[:16], B, T, H, 128, 128, 0, 0, P((1 << 40) * 20), 1 << 45, None) == 2


def test_bwd_gate_forms_on_the_host(lib):
    # scalar beta implies w: passing w or dw with GDN2_BETA_SCALAR is refused; an unknown flag is
    # refused; the workspace query grows for scalar gates (repeated gates and their per-channel
    # gradients) and for the L2 norm (row norms)
    far = [P((1 << 40) * (i + 1)) for i in range(16)]
    ws = P((1 << 40) * 20)
    f = lib.gdn2_chunk_bwd
    q = lib.gdn2_chunk_bwd_workspace_bytes
    B, T, H = 1, 64, 2
    assert f(*far[:16], B, T, H, 64, 64, 0, 2, ws, 1 << 30, None) == 3           # w given
    p = list(far[:16])
    p[5] = None
    assert f(*p, B, T, H, 64, 64, 0, 2, ws, 1 << 30, None) == 3                  # dw given
    assert f(*far[:16], B, T, H, 64, 64, 0, 16, ws, 1 << 30, None) == 3          # unknown flag
    assert q(B, T, H, 64, 64, 0, 3) > q(B, T, H, 64, 64, 0, 1) > q(B, T, H, 64, 64, 0, 0) > 0
    assert q(B, T, H, 64, 64, 0, 4) > q(B, T, H, 64, 64, 0, 0) == q(B, T, H, 64, 64, 0, 8)


def test_saved_training_step_rejects_bad_arguments(lib):
    # gdn2_chunk_fwd_save and gdn2_chunk_bwd_saved, refused on the host before any launch: the
    # saving forward takes what the backward takes (bf16, d_k == d_v <= 128) and needs the
    # backward's workspace; the saved backward checks as gdn2_chunk_bwd
    far = [P((1 << 40) * (i + 1)) for i in range(16)]
    ws = P((1 << 40) * 20)
    fs, bs = lib.gdn2_chunk_fwd_save, lib.gdn2_chunk_bwd_saved
    need = lib.gdn2_chunk_bwd_workspace_bytes(1, 64, 2, 64, 64, 0, 0)
    assert need > 0
    assert fs(*far[:9], 1, 64, 2, 64, 64, 0, 0, None, 0, None) == 7                  # no workspace
    assert fs(*far[:9], 1, 64, 2, 64, 64, 0, 0, ws, need - 1, None) == 7             # too small
    assert fs(*far[:9], 1, 64, 2, 64, 64, 0, 0, P((1 << 40) * 20 + 16), need, None) == 4  # misaligned
    assert fs(*far[:9], 1, 64, 2, 64, 64, 1, 0, ws, 1 << 30, None) == 3              # fp32 inputs
    assert fs(*far[:9], 1, 64, 2, 256, 256, 0, 0, ws, 1 << 30, None) == 3            # head size 256
    assert fs(*far[:9], 1, 64, 2, 64, 32, 0, 0, ws, 1 << 30, None) == 3              # d_k != d_v
    assert fs(*far[:9], 1, 64, 2, 64, 64, 0, 16, ws, 1 << 30, None) == 3             # unknown flag
    p = list(far[:9])
    p[7] = None
    assert fs(*p, 1, 64, 2, 64, 64, 0, 0, ws, 1 << 30, None) == 1                    # no o
    assert fs(*far[:9], 1, 64, 2, 64, 64, 0, 0, far[0], 1 << 30, None) == 5          # workspace on q
    assert bs(*far[:16], 1, 64, 2, 64, 64, 0, 0, None, 0, None) == 7                 # no workspace
    assert bs(*far[:16], 1, 64, 2, 64, 64, 0, 2, ws, 1 << 30, None) == 3             # w with scalar beta
    assert bs(*far[:16], 1, 64, 2, 64, 64, 1, 0, ws, 1 << 30, None) == 3             # fp32 inputs
    # the packed pair: cu_seqlens required; the saving forward takes the backward's workspace size
    fv, bv = lib.gdn2_chunk_fwd_varlen_save, lib.gdn2_chunk_bwd_varlen_saved
    cu = P((1 << 40) * 30)
    vneed = lib.gdn2_chunk_bwd_varlen_workspace_bytes(3, 200, 2, 64, 64, 0, 0)
    assert vneed > 0
    assert fv(*far[:9], None, 3, 200, 2, 64, 64, 0, 0, ws, 1 << 30, None) == 1       # no cu_seqlens
    assert fv(*far[:9], cu, 3, 200, 2, 64, 64, 0, 0, None, 0, None) == 7             # no workspace
    assert fv(*far[:9], cu, 3, 200, 2, 64, 64, 0, 0, ws, vneed - 1, None) == 7       # too small
    assert fv(*far[:9], cu, 3, 200, 2, 64, 64, 1, 0, ws, 1 << 30, None) == 3         # fp32 inputs
    assert fv(*far[:9], cu, 0, 200, 2, 64, 64, 0, 0, ws, 1 << 30, None) == 2         # no sequences
    assert bv(*far[:16], None, 3, 200, 2, 64, 64, 0, 0, ws, 1 << 30, None) == 1      # no cu_seqlens
    assert bv(*far[:16], cu, 3, 200, 2, 64, 64, 0, 0, None, 0, None) == 7            # no workspace


def test_bwd_varlen_rejects_bad_arguments(lib):
    # every call below is refused on the host before any launch
    far = [P((1 << 40) * (i + 1)) for i in range(16)]
    cu = P((1 << 40) * 17)
    ws = P((1 << 40) * 20)
    f = lib.gdn2_chunk_bwd_varlen
    qs = lib.gdn2_chunk_bwd_varlen_workspace_bytes
    need = qs(4, 1000, 2, 128, 128, 0, 0)
    assert need > 0
    assert qs(8, 1000, 2, 128, 128, 0, 0) > need       # more sequences: a larger chunk bound
    assert qs(4, 1000, 2, 128, 128, 0, 3) > need       # scalar gates: repeated gates and gradients
    assert qs(4, 1000, 2, 128, 128, 1, 0) == 0         # fp32 inputs
    assert qs(0, 1000, 2, 128, 128, 0, 0) == 0
    assert qs(4, 0, 2, 128, 128, 0, 0) == 0            # no rows: no workspace

    def call(ptrs=far, cu=cu, N=4, T=1000, H=2, dk=128, dv=128, dt=0, flags=0, ws=ws, wsb=need):
        return f(*ptrs, cu, N, T, H, dk, dv, dt, flags, ws, wsb, None)

    assert call(N=0) == 2
    assert call(T=-1) == 2
    assert call(cu=None) == 1
    assert call(cu=P((1 << 40) * 17 + 2)) == 4
    assert call(ws=None) == 7
    assert call(wsb=need - 1) == 7
    assert call(ws=P((1 << 40) * 20 + 128)) == 4        # workspace not 256-byte aligned
    assert call(dk=256, dv=256) == 3
    assert call(dt=1) == 3
    assert call(flags=16) == 3
    assert call(flags=2) == 3                           # scalar beta with w and dw given
    assert call(cu=far[9]) == 5                         # cu_seqlens overlaps dq
    assert call(ws=far[12]) == 5                        # workspace over db
    assert call(N=32, T=64 * 1024 * 32, H=64, wsb=1 << 45) == 2  # grid past 2^31 threads


def test_rmsnorm_rejects_bad_arguments(lib):
    # every call below is refused on the host (or has nothing to do) before any launch
    far = [P((1 << 40) * (i + 1)) for i in range(8)]
    fwd, bwd, qs = lib.gdn2_rmsnorm_fwd, lib.gdn2_rmsnorm_bwd, lib.gdn2_rmsnorm_bwd_workspace_bytes
    x, w, y = far[0], far[1], far[2]
    assert fwd(x, w, y, -1, 128, 1e-6, 1, None) == 2
    assert fwd(x, w, y, 10, 48, 1e-6, 1, None) == 3
    assert fwd(x, w, y, 10, 128, 1e-6, 5, None) == 3          # unknown output dtype
    assert fwd(x, w, y, 10, 128, -1.0, 1, None) == 3          # eps < 0
    assert fwd(x, w, y, 10, 128, float("inf"), 1, None) == 3
    assert fwd(x, w, y, 10, 128, float("nan"), 1, None) == 3
    assert fwd(x, w, y, 0, 128, 1e-6, 1, None) == 0           # no rows: nothing enqueued
    assert fwd(None, w, y, 10, 128, 1e-6, 1, None) == 1
    assert fwd(P((1 << 40) + 8), w, y, 10, 128, 1e-6, 1, None) == 4
    assert fwd(x, w, x, 10, 128, 1e-6, 0, None) == 5          # in place only with float32 output
    assert fwd(x, w, P((1 << 40) + 512), 10, 128, 1e-6, 1, None) == 5  # partial overlap with x
    assert fwd(x, w, P((1 << 40) * 2 - 256), 10, 128, 1e-6, 1, None) == 5  # y runs into weight
    assert fwd(x, w, y, 1 << 36, 128, 1e-6, 1, None) == 2    # grid past 2^31 threads
    # backward: dweight partials, one [d] row per workgroup step of 4096 / d rows, at most 1024
    assert qs(1000, 128) == 32 * 128 * 4
    assert qs(10 ** 7, 128) == 1024 * 128 * 4
    assert qs(10, 48) == 0 and qs(-1, 128) == 0
    dy, dx, dw, ws = far[3], far[4], far[5], far[6]
    need = qs(1000, 128)
    assert bwd(x, w, dy, dx, dw, 1000, 128, 1e-6, None, 0, None) == 7
    assert bwd(x, w, dy, dx, dw, 1000, 128, 1e-6, ws, need - 1, None) == 7
    assert bwd(x, w, dy, dx, dw, 1000, 128, -1.0, ws, need, None) == 3
    assert bwd(x, w, None, dx, dw, 1000, 128, 1e-6, ws, need, None) == 1
    assert bwd(x, w, dy, x, dw, 1000, 128, 1e-6, ws, need, None) == 5      # dx over x
    assert bwd(x, w, dy, dx, dy, 1000, 128, 1e-6, ws, need, None) == 5     # dweight over dy
    assert bwd(x, w, dy, dx, dw, 1000, 128, 1e-6, dx, need, None) == 5     # workspace over dx
    assert bwd(x, w, dy, dx, None, 0, 128, 1e-6, None, 0, None) == 0       # nothing to do
    # the allocation-free variant: the same argument checks, without a workspace argument
    na = lib.gdn2_rmsnorm_bwd_noalloc
    assert na(x, w, dy, dx, dw, -1, 128, 1e-6, None) == 2
    assert na(x, w, dy, dx, dw, 1000, 48, 1e-6, None) == 3
    assert na(x, w, dy, dx, dw, 1000, 128, float("nan"), None) == 3
    assert na(x, w, None, dx, dw, 1000, 128, 1e-6, None) == 1
    assert na(x, w, dy, P((1 << 40) * 5 + 8), dw, 1000, 128, 1e-6, None) == 4
    assert na(x, w, dy, x, dw, 1000, 128, 1e-6, None) == 5                 # dx over x
    assert na(x, w, dy, dx, dy, 1000, 128, 1e-6, None) == 5                # dweight over dy
    assert na(x, w, dy, dx, None, 0, 128, 1e-6, None) == 0                 # nothing to do


def test_sdm_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    x, c1, c2, idx, wt = P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000)
    a = lib.gdn2_sdm_address
    assert a(x, c1, c2, -1, 2, 128, 256, 64, 0, idx, wt, None) == 2       # rows < 0
    assert a(x, c1, c2, 4, 2, 96, 256, 64, 0, idx, wt, None) == 3         # d_k
    assert a(x, c1, c2, 4, 2, 128, 100, 64, 0, idx, wt, None) == 3        # n not a power of two in range
    assert a(x, c1, c2, 4, 2, 128, 64, 65, 0, idx, wt, None) == 3         # m > 64
    assert a(x, c1, c2, 4, 2, 128, 64, 0, 0, idx, wt, None) == 3          # m = 0
    assert a(x, None, c2, 4, 2, 128, 64, 8, 0, idx, wt, None) == 1
    assert a(P(0x10004), c1, c2, 4, 2, 128, 64, 8, 0, idx, wt, None) == 4
    assert a(x, c1, c2, 4, 2, 128, 64, 8, 0, P(0x10000), wt, None) == 5   # idx over x
    assert a(x, c1, c2, 0, 2, 128, 64, 8, 0, None, None, None) == 0       # no rows: nothing to do
    f = lib.gdn2_sdm_fwd
    p = [P(0x100000 * (i + 1)) for i in range(12)]  # v, alpha, b, w, widx, wwt, ridx, rwt, M, stamp, L, o

    def call(*ptrs, B=2, T=3, H=2, N=4096, dv=128, W=64, R=64, dt=0):
        return f(*ptrs, B, T, H, N, dv, W, R, dt, None)
    assert call(*p, dv=96) == 3
    assert call(*p, W=65) == 3 and call(*p, R=0) == 3
    assert call(*p, N=32) == 2                       # W > N
    assert call(*p, N=0) == 2 and call(*p, N=1 << 31) == 2
    assert call(*p, T=-1) == 2
    q = list(p)
    q[0] = None
    assert call(*q) == 1
    q = list(p)
    q[8] = P(0x100008)
    assert call(*q) == 4
    q = list(p)
    q[11] = p[10]                                    # o over L
    assert call(*q) == 5
    q = list(p)
    q[9] = p[0]                                      # stamp over v
    assert call(*q) == 5
    q = list(p)
    q[10] = None
    assert call(*q) == 1
    assert call(*p, T=0) == 0 and call(*p, B=0) == 0
    fo = lib.gdn2_sdm_fold
    assert fo(p[8], p[9], p[10], 2, 2, 4096, 96, None) == 3
    assert fo(None, p[9], p[10], 2, 2, 4096, 128, None) == 1
    assert fo(p[8], p[8], p[10], 2, 2, 4096, 128, None) == 5
    assert fo(p[8], p[9], p[10], 0, 2, 4096, 128, None) == 0
