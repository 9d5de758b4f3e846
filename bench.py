#!/usr/bin/env python3
"""Benchmark: Gated DeltaNet-2 chunkwise prefill tokens/s and decode-state HBM GB/s on one GPU.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Prefill workload: one 1.3B-scale layer, B=8, H=16, T=4096, d_k=d_v=128 (262,144 state floats
per batch element), bf16 q/k/v/alpha/b/w, fp32 S0 ~ N(0, 0.1^2), fp32 o and final state.
Synthetic seeded inputs (no datasets or weights), resident in HBM before timing starts.
A timed step is one gdn2_chunk_fwd call over the whole batch; `value` = B*T / (step time).

Decode workload (reported beside it): B=256 (and B=1024, whose 1 GiB state cannot sit in
the 256 MB Infinity Cache), H=16, d=128, fp32 state updated in place over consecutive steps.

Prints ONE JSON line. `roofline` is for the prefill call (with a workspace: the prep kernel and
the chain kernel that one gdn2_chunk_fwd call enqueues): algorithmic bytes per call over the
call's average duration (HIP events on the launch stream) against 8 TB/s HBM3E; `traffic` is
the HBM bytes per call that rocprofv3 counted for the same kernels.
`cpu_baseline` times the fp64 oracle (tests-only code, timed here as a reported baseline) on a
bounded sample of the same workload with all host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3

CSRC = os.path.join(ROOT, "gated_delta_rule_25_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


IMPL_SOURCES = {"split": "chunk_split.hip", "fused": "chunk_fused.hip", "recurrent": "recurrent.hip"}


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with runs of whitespace collapsed: two sources that
    differ only in comments or layout compile to the same code and get the same digest."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":  # a string or character literal, copied whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_digest(impl: str) -> str:
    """sha256 over the code (comments and layout aside) of the sources that the impl's kernels are
    built from: its .hip file under csrc/ and every csrc/ header it includes, directly or through
    another header, in name order. It names the build that a profile's counters were taken on."""
    import hashlib
    import re
    seen, todo = set(), [IMPL_SOURCES[impl]]
    while todo:
        name = todo.pop()
        if name in seen or not os.path.isfile(os.path.join(CSRC, name)):
            continue
        seen.add(name)
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            todo += re.findall(r'^\s*#\s*include\s+"([^"]+)"', f.read(), flags=re.M)
    h = hashlib.sha256()
    for name in sorted(seen):
        h.update(name.encode() + b"\0")
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(impl: str, digest: str):
    """HBM bytes per gdn2_chunk_fwd call at B8 H16 T4096 d128 bf16 that a summary in profiles/
    states for these exact kernel sources (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated),
    from its line "bench-traffic: impl=<impl> bytes=<n> sources=<digest>". None when no summary
    was taken on these sources: counters of another build say nothing about this one."""
    if not os.path.isdir(PROFILES):
        return None
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith((".txt", ".md")):
            continue
        with open(os.path.join(PROFILES, name), encoding="utf-8") as f:
            for line in f:
                if not line.startswith("bench-traffic:"):
                    continue
                kv = dict(x.split("=", 1) for x in line.split()[1:] if "=" in x)
                if kv.get("impl") == impl and kv.get("sources") == digest:
                    return float(kv["bytes"])
    return None


def prefill_bytes_per_head_token(dk: int, dv: int, T: int, es: int = 2) -> float:
    # q, k, alpha, b + v, w (es bytes each: 2 for bf16, 4 for fp32) + o (fp32) + S0 read and S_T
    # write amortised over T
    return 4 * dk * es + 2 * dv * es + 4 * dv + 8 * dk * dv / T


def prefill_flops_per_head_token(dk: int, dv: int, C: int = 64) -> float:
    # three state products (W S, Q_hat S, K_bar^T Delta) + five triangular C x C products
    # (A, P, W = T E_hat, U~ = T U, P Delta; counted at half) + the UT solve
    return 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3


KERNELS = {
    "split": "prep_kernel + chain_kernel (one gdn2_chunk_fwd call with the two-kernel workspace)",
    "fused": "fused_kernel (one gdn2_chunk_fwd call without a workspace: allocation-free)",
    "recurrent": "recurrent_kernel (gdn2_recurrent_fwd)",
}


def prefill_kwargs(g, impl, B, T, H, dk, dv, ring_mb=None, dtype=None):
    """Keyword arguments of chunk_fwd for one schedule, with any workspace allocated up front so
    that no allocation falls inside a timed region."""
    import torch
    if impl == "recurrent":
        return {}
    dtype = torch.bfloat16 if dtype is None else dtype
    kw = dict(schedule=impl)
    if impl == "split":
        need = g.chunk_fwd_workspace_bytes(B, T, H, dk, dv, dtype=dtype)
        if need and ring_mb is not None:
            state = B * H * dk * dv * 4
            per_chunk = g.chunk_fwd_workspace_bytes(B, 64, H, dk, dv, dtype=dtype) - state
            slots = max(1, int(ring_mb * 2**20) // per_chunk)
            need = min(need, state + slots * per_chunk)
        if need:
            kw["workspace"] = torch.empty(need, device="cuda", dtype=torch.uint8)
    return kw


def decode_bytes_per_head(dk: int, dv: int) -> float:
    return 2 * 4 * dk * dv + 4 * dk * 2 + 2 * dv * 2 + 4 * dv


def time_prefill(g, ins, steps, warmup, impl, ring_mb=None, **flags):
    import torch
    fn = g.recurrent_fwd if impl == "recurrent" else g.chunk_fwd
    args = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    B, T, H, dk = ins["q"].shape
    dv = ins["v"].shape[-1]
    o = torch.empty(B, T, H, dv, device="cuda", dtype=torch.float32)
    S_out = torch.empty(B, H, dk, dv, device="cuda", dtype=torch.float32)
    kw = dict(o=o, S_out=S_out, **prefill_kwargs(g, impl, B, T, H, dk, dv, ring_mb, ins["q"].dtype))
    kw.update(flags)
    for _ in range(warmup):
        fn(*args, ins["S0"], **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        fn(*args, ins["S0"], **kw)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    return wall, kern_ms


def time_prefill_cold(g, ins, reps, impl):
    """Per-call kernel time with a 512 MiB scrub written between calls (evicts the 256 MB
    Infinity Cache and the L2s), on the launch stream."""
    import torch
    args = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    B, T, H, dk = ins["q"].shape
    dv = ins["v"].shape[-1]
    o = torch.empty(B, T, H, dv, device="cuda", dtype=torch.float32)
    S_out = torch.empty(B, H, dk, dv, device="cuda", dtype=torch.float32)
    kw = dict(o=o, S_out=S_out, **prefill_kwargs(g, impl, B, T, H, dk, dv, dtype=ins["q"].dtype))
    fn = g.recurrent_fwd if impl == "recurrent" else g.chunk_fwd
    scrub = torch.empty(1 << 27, device="cuda", dtype=torch.float32)  # 512 MiB
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(reps + 1):
        scrub.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*args, ins["S0"], **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        if i:
            ms.append(e0.elapsed_time(e1))
    del scrub
    return sum(ms) / len(ms)


def prefill_leg(g, name, steps, impl):
    """One more prefill workload, timed like the headline one (warm, back to back)."""
    import torch
    from gated_delta_rule_25_amd.inputs import WORKLOADS, make_inputs_torch
    wl = WORKLOADS[name]
    ins = make_inputs_torch(wl, device="cuda")
    torch.cuda.synchronize()
    _, kern_ms = time_prefill(g, ins, steps, 1, impl)
    avg = sum(kern_ms) / len(kern_ms)
    head_tokens = wl.B * wl.T * wl.H
    fp32 = wl.dtype == "fp32"
    alg = prefill_bytes_per_head_token(wl.d_k, wl.d_v, wl.T, 4 if fp32 else 2) * head_tokens
    res = dict(config=f"B{wl.B} H{wl.H} T{wl.T} d{wl.d_k} {wl.dtype} gates={wl.gates}",
               kernel_ms=round(avg, 4), tokens_per_s=round(wl.B * wl.T / (avg * 1e-3), 1))
    if wl.gates == "general":  # (scalar gates move fewer input bytes; no byte roofline quoted)
        res.update(gbs=round(alg / (avg * 1e-3) / 1e9, 1),
                   frac=round(alg / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    if fp32:  # fp32 operands run at the fp32 matrix-core rate, which bounds this path before HBM
        tf = prefill_flops_per_head_token(wl.d_k, wl.d_v) * head_tokens / (avg * 1e-3) / 1e12
        res.update(mfma_f32_tflops=round(tf, 1), mfma_f32_frac=round(tf / MFMA_F32_PEAK_TFLOPS, 4))
    print(f"[bench] {name}: {avg:.3f} ms/launch, {res['tokens_per_s']:.3e} tokens/s", file=sys.stderr,
          flush=True)
    del ins
    torch.cuda.empty_cache()
    return res


def varlen_leg(g, steps, ref_ms=None):
    """gdn2_chunk_fwd_varlen on a packed batch with the headline's token count: 32 sequences in a
    length mix (packed_lengths), 32,768 rows, H16 d128 bf16; warm, back to back, on the launch
    stream. ref_ms: the equal-length B8 T4096 call, for the ratio."""
    import torch
    from gated_delta_rule_25_amd.inputs import WORKLOADS, make_packed_inputs, packed_lengths
    wl = WORKLOADS["prefill_1p3b"]
    lengths = packed_lengths(32, 32768, seed=wl.seed)
    ins = make_packed_inputs(wl, lengths, device="cuda")
    H, dk, dv = wl.H, wl.d_k, wl.d_v
    T = sum(lengths)
    o = torch.empty(T, H, dv, device="cuda", dtype=torch.float32)
    S_out = torch.empty(len(lengths), H, dk, dv, device="cuda", dtype=torch.float32)
    ws = torch.empty(g.chunk_fwd_varlen_workspace_bytes(len(lengths), T, H, dk, dv), dtype=torch.uint8,
                     device="cuda")
    args = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w")] + [ins["cu_seqlens"], ins["S0"]]
    kw = dict(o=o, S_out=S_out, workspace=ws)
    g.chunk_fwd_varlen(*args, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.chunk_fwd_varlen(*args, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = sum(prefill_bytes_per_head_token(dk, dv, L) * L * H for L in lengths if L > 0)
    res = dict(config=f"32 sequences packed, {T} rows, lengths {min(lengths)}..{max(lengths)}, H{H} d{dk} bf16",
               ms=round(ms, 4), tokens_per_s=round(T / (ms * 1e-3), 1), algorithmic_bytes=int(alg),
               gbs=round(alg / (ms * 1e-3) / 1e9, 1), frac=round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               vs_equal_length=(round(ms / ref_ms, 3) if ref_ms else None))
    print(f"[bench] packed prefill: {ms:.3f} ms/call, {res['tokens_per_s']:.3e} tokens/s, {res['gbs']} GB/s "
          f"algorithmic", file=sys.stderr, flush=True)
    del ins, o, S_out, ws
    torch.cuda.empty_cache()
    return res


def bwd_bytes_per_head_token(dk: int, dv: int, T: int) -> float:
    # q, k, alpha, b, v, w (bf16) + dO (fp32) read; dq, dk, dalpha, db, dv, dw (fp32) written;
    # S0 and dS_T read and dS0 written, amortised over T
    return 4 * dk * 2 + 2 * dv * 2 + 4 * dv + 4 * dk * 4 + 2 * dv * 4 + 12 * dk * dv / T


def backward_leg(g, steps):
    """gdn2_chunk_bwd at the prefill shape (B8 H16 T4096 d128 bf16), warm, back to back, on the
    launch stream."""
    import torch
    from gated_delta_rule_25_amd.inputs import WORKLOADS, make_cotangents, make_inputs_torch
    wl = WORKLOADS["prefill_1p3b"]
    ins = make_inputs_torch(wl, device="cuda")
    cot = make_cotangents(wl, device="cuda")
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.d_k, wl.d_v
    ws = torch.empty(g.chunk_bwd_workspace_bytes(B, T, H, dk, dv), dtype=torch.uint8, device="cuda")
    out = {}
    args = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w", "S0")] + [cot["dO"], cot["dS_T"]]
    out = g.chunk_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.chunk_bwd(*args, workspace=ws, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = bwd_bytes_per_head_token(dk, dv, T) * B * T * H
    res = dict(config=f"B{B} H{H} T{T} d{dk} bf16 gates=general", ms=round(ms, 4),
               tokens_per_s=round(B * T / (ms * 1e-3), 1), algorithmic_bytes=int(alg),
               gbs=round(alg / (ms * 1e-3) / 1e9, 1), frac=round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               workspace_bytes=int(ws.numel()))

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / n

    # the same shape with the prologue flags (inputs taken as raw q, k and gate pre-activations)
    res["prologue_ms"] = round(timed(lambda: g.chunk_bwd(*args, l2norm=True, gate_logits=True), max(2, steps // 2)), 4)
    # Gated DeltaNet form: scalar alpha and beta (the per-head first channel of the general gates)
    sa = ins["alpha"][..., 0].contiguous()
    sb = ins["b"][..., 0].contiguous()
    sargs = [ins["q"], ins["k"], ins["v"], sa, sb, None, ins["S0"], cot["dO"], cot["dS_T"]]
    res["scalar_gates_ms"] = round(timed(lambda: g.chunk_bwd(*sargs), max(2, steps // 2)), 4)
    del sa, sb, sargs
    # packed batch: the same rows as 32 sequences in a length mix (gdn2_chunk_bwd_varlen)
    from gated_delta_rule_25_amd.inputs import make_packed_inputs, packed_lengths
    lengths = packed_lengths(32, B * T, seed=wl.seed)
    pk = make_packed_inputs(wl, lengths, device="cuda")
    pdO = cot["dO"].reshape(B * T, H, dv)
    pdS = torch.randn(len(lengths), H, dk, dv, device="cuda")
    pws = torch.empty(g.chunk_bwd_varlen_workspace_bytes(len(lengths), B * T, H, dk, dv), dtype=torch.uint8,
                      device="cuda")
    pargs = [pk[n] for n in ("q", "k", "v", "alpha", "b", "w")] + [pk["cu_seqlens"], pk["S0"], pdO, pdS]
    res["packed_ms"] = round(timed(lambda: g.chunk_bwd_varlen(*pargs, workspace=pws), max(2, steps // 2)), 4)
    del pk, pdO, pdS, pws, pargs
    # a training step without the recomputation: the forward that saves into the backward's
    # workspace (gdn2_chunk_fwd_save), then the backward that reads the saves (gdn2_chunk_bwd_saved);
    # against it, the forward with its own workspace (gdn2_chunk_fwd) then gdn2_chunk_bwd
    fargs = args[:7]
    o = torch.empty(B, T, H, dv, device="cuda")
    S_T = torch.empty(B, H, dk, dv, device="cuda")
    fws = torch.empty(g.chunk_fwd_workspace_bytes(B, T, H, dk, dv), dtype=torch.uint8, device="cuda")
    res["fwd_save_ms"] = round(timed(lambda: g.chunk_fwd_save(*fargs, o=o, S_out=S_T, workspace=ws), max(2, steps // 2)), 4)
    res["bwd_saved_ms"] = round(timed(lambda: g.chunk_bwd(*args, saved=ws, out=out), steps), 4)
    res["train_step_saved_ms"] = round(timed(lambda: (g.chunk_fwd_save(*fargs, o=o, S_out=S_T, workspace=ws),
                                                      g.chunk_bwd(*args, saved=ws, out=out)), max(2, steps // 2)), 4)
    res["train_step_recompute_ms"] = round(timed(lambda: (g.chunk_fwd(*fargs, o=o, S_out=S_T, workspace=fws),
                                                          g.chunk_bwd(*args, workspace=ws, out=out)), max(2, steps // 2)), 4)
    del o, S_T, fws
    print(f"[bench] backward: {ms:.3f} ms/call, {res['tokens_per_s']:.3e} tokens/s, {res['gbs']} GB/s "
          f"algorithmic ({100 * res['frac']:.1f}% of HBM); with the prologue {res['prologue_ms']:.3f} ms, "
          f"scalar gates {res['scalar_gates_ms']:.3f} ms, packed (32 sequences) {res['packed_ms']:.3f} ms; "
          f"saved forward {res['fwd_save_ms']:.3f} ms + saved backward {res['bwd_saved_ms']:.3f} ms "
          f"(step {res['train_step_saved_ms']:.3f} ms against {res['train_step_recompute_ms']:.3f} ms recomputing)",
          file=sys.stderr, flush=True)
    del ins, cot, ws, out
    torch.cuda.empty_cache()
    return res


def rmsnorm_leg(g, steps):
    """gdn2_rmsnorm_fwd / _bwd on the o of the B8 H16 T4096 d128 prefill (524,288 rows of 128
    fp32): forward to fp32 and to bf16, backward with dweight; warm, back to back. Algorithmic
    bytes per row: x read + y written (4 d + 4 d, or 4 d + 2 d for bf16); backward x, dy read and
    dx written (12 d)."""
    import torch
    rows, d = 8 * 4096 * 16, 128
    gen = torch.Generator(device="cuda").manual_seed(20256)
    x = torch.randn(rows, d, device="cuda", generator=gen)
    dy = torch.randn(rows, d, device="cuda", generator=gen)
    w = torch.randn(d, device="cuda", generator=gen)
    y = torch.empty_like(x)
    y16 = torch.empty(rows, d, device="cuda", dtype=torch.bfloat16)
    dx = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / steps

    res = dict(config=f"{rows} rows x {d} fp32 (o of B8 H16 T4096)")
    for name, fn, nbytes in (("fwd_f32", lambda: g.rmsnorm_fwd(x, w, out=y), 8 * d),
                             ("fwd_bf16", lambda: g.rmsnorm_fwd(x, w, out=y16), 6 * d),
                             ("bwd", lambda: g.rmsnorm_bwd(x, w, dy, dx=dx), 12 * d)):
        ms = timed(fn)
        gbs = nbytes * rows / (ms * 1e-3) / 1e9
        res[name] = dict(ms=round(ms, 4), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
    print("[bench] output RMS norm: " + ", ".join(f"{n} {res[n]['ms']:.4f} ms ({res[n]['gbs']} GB/s)"
                                                 for n in ("fwd_f32", "fwd_bf16", "bwd")),
          file=sys.stderr, flush=True)
    del x, dy, w, y, y16, dx
    torch.cuda.empty_cache()
    return res


def sdm_leg(g, steps):
    """Sparse delta memory at B8 H16, N = 65,536 slots of d_v = 128 per head (32 MiB; 4 GiB in all),
    W = R = 64: one decode step (gdn2_sdm_fwd with T = 1), the product-key addressing of a
    B8 T4096 prefill's keys (524,288 queries, gdn2_sdm_address), and a 256-token token-by-token
    prefill. Bytes per head-token: the W write slots read and written and the R read slots read
    (3 x 64 x 128 x 4 B = 96 KiB) plus the token's inputs."""
    import torch
    from gated_delta_rule_25_amd.inputs import make_sdm_inputs
    B, H, n, dv, W = 8, 16, 256, 128, 64
    N = n * n
    stream = torch.cuda.current_stream()

    def timed(fn, k):
        fn()
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / k

    gen = torch.Generator(device="cuda").manual_seed(20257)
    state = g.sdm_state(torch.randn(B, H, N, dv, device="cuda", generator=gen) * 0.1)
    res = dict(config=f"B{B} H{H} N={N} slots x d_v={dv} fp32 (memory {B * H * N * dv * 4 >> 30} GiB), W=R={W}")
    dec = make_sdm_inputs(B, 64, H, 128, dv, n, W, W, seed=20258, with_memory=False, device="cuda")
    pool = [{k: dec[k][:, i:i + 1].contiguous() for k in ("v", "alpha", "b", "w", "widx", "wwt", "ridx", "rwt")}
            for i in range(64)]
    it = [0]

    def step():
        x = pool[it[0] % 64]
        it[0] += 1
        g.sdm_fwd(x["v"], x["alpha"], x["b"], x["w"], x["widx"], x["wwt"], x["ridx"], x["rwt"], state)
    ms = timed(step, steps)
    # the same steps replayed from a HIP graph of 64 steps: the device's time per step, without
    # the host's cost per call (a serving loop would capture its steps the same way)
    ms_graph = None
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(3):
                step()
        stream.wait_stream(side)
        with torch.cuda.graph(graph):
            for _ in range(64):
                step()
        ms_graph = timed(graph.replay, max(2, steps // 64)) / 64
        del graph
    except RuntimeError as e:  # capture unavailable: report the per-call time only
        print(f"[bench] sdm decode graph capture failed: {e}", file=sys.stderr, flush=True)
    # W rows read and written, R rows read (fp32), their stamps (fp64; W written), the token's
    # v and w (bf16), alpha and b, the 2 x 64 slot indices and weights, o written (fp32)
    per_ht = 3 * W * dv * 4 + 3 * W * 8 + dv * 2 * 2 + 2 * 2 + 2 * W * 8 + dv * 4
    gbs = per_ht * B * H / (ms * 1e-3) / 1e9
    res["decode"] = dict(us_per_step=round(ms * 1e3, 2), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                         head_tokens_per_s=round(B * H / (ms * 1e-3), 1))
    if ms_graph is not None:
        gg = per_ht * B * H / (ms_graph * 1e-3) / 1e9
        res["decode"].update(graph_us_per_step=round(ms_graph * 1e3, 2), graph_gbs=round(gg, 1),
                             graph_frac=round(gg / HBM_PEAK_GBS, 4))
    del dec, pool
    T = 4096
    ad = make_sdm_inputs(B, T, H, 128, dv, n, 1, 1, seed=20259, with_memory=False, device="cuda")
    ms = timed(lambda: g.sdm_address(ad["k"], ad["C1"], ad["C2"], W), max(2, steps // 20))
    res["address"] = dict(queries=B * T * H, ms=round(ms, 4), queries_per_s=round(B * T * H / (ms * 1e-3), 1))
    del ad
    Tp = 256
    pf = make_sdm_inputs(B, Tp, H, 128, dv, n, W, W, seed=20260, with_memory=False, device="cuda")
    ms = timed(lambda: g.sdm_fwd(pf["v"], pf["alpha"], pf["b"], pf["w"], pf["widx"], pf["wwt"], pf["ridx"],
                                 pf["rwt"], state), 2)
    gbs = per_ht * B * H * Tp / (ms * 1e-3) / 1e9
    res["prefill"] = dict(T=Tp, ms=round(ms, 4), us_per_token=round(ms * 1e3 / Tp, 3), gbs=round(gbs, 1),
                          tokens_per_s=round(B * Tp / (ms * 1e-3), 1))
    print(f"[bench] sdm: decode {res['decode']['us_per_step']} us/step ({res['decode']['gbs']} GB/s; from a graph "
          f"{res['decode'].get('graph_us_per_step')} us/step), "
          f"address {res['address']['ms']} ms for {B * T * H} queries, prefill {res['prefill']['us_per_token']} "
          f"us/token", file=sys.stderr, flush=True)
    del pf, state
    torch.cuda.empty_cache()
    return res


def time_decode(g, B, H, d, steps, warmup, seed):
    import torch
    from gated_delta_rule_25_amd.inputs import make_decode_inputs
    pool = min(steps, 64)
    ins = make_decode_inputs(B, H, d, d, pool, seed=seed, device="cuda", generator="torch")
    S = ins["S0"].clone()
    o = torch.empty(B, H, d, device="cuda", dtype=torch.float32)
    xs = [ins[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    for i in range(warmup):
        g.decode_step(*[x[i % pool] for x in xs], S, o=o)
    S.copy_(ins["S0"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    step_in = [[x[i % pool] for x in xs] for i in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        g.decode_step(*step_in[i], S, o=o)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    del ins, S, o, xs, step_in
    return wall, kern_ms


def cpu_baseline(ins_gpu, n_heads: int):
    """Time the fp64 oracle on n_heads full-length (b, h) sequences of the same inputs."""
    import torch

    import oracle
    B, T, H, dk = ins_gpu["q"].shape
    sel = [(i // H, i % H) for i in range(n_heads)]

    def pick(x, tok=True):
        if tok:
            return torch.stack([x[b, :, h] for b, h in sel])[:, :, None].cpu()
        return torch.stack([x[b, h] for b, h in sel])[:, None].cpu()

    sub = {n: pick(ins_gpu[n]) for n in ("q", "k", "v", "alpha", "b", "w")}
    S0 = pick(ins_gpu["S0"], tok=False)
    threads = oracle.default_threads()
    q, k, v, a, b, w = (oracle._f64(sub[n]) for n in ("q", "k", "v", "alpha", "b", "w"))
    S0 = oracle._f64(S0)
    t0 = time.perf_counter()
    oracle.forward(q, k, v, a, b, w, S0, threads=threads)
    dt = time.perf_counter() - t0
    head_tokens_per_s = n_heads * T / dt
    return dict(value=head_tokens_per_s / H, unit="tokens/s", cores=min(threads, n_heads),
                kind="oracle",
                sample=f"{n_heads} of {B * H} (b,h) sequences at full T={T}, d={dk}; "
                       f"{dt:.2f} s wall; tokens/s = head-tokens/s / H (H={H})")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--impl", choices=["split", "fused", "recurrent"], default="split",
                    help="split: two-kernel chunkwise path (with its workspace, the fastest); fused: "
                         "fused chunkwise kernel (no workspace, allocation-free); recurrent: "
                         "token-by-token kernel")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=128)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for HBM byte "
                         "counters)")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-backward", action="store_true", help="skip the backward (gdn2_chunk_bwd) leg")
    ap.add_argument("--skip-others", action="store_true",
                    help="skip the long-context and scalar-gate prefill legs")
    ap.add_argument("--workload", default="prefill_1p3b",
                    choices=["prefill_1p3b", "long_prefill", "gdn_scalar", "kda_scalar"],
                    help="prefill input recipe to time (the headline figure uses prefill_1p3b)")
    ap.add_argument("--ring-mb", type=float, default=None,
                    help="size the two-kernel path's workspace ring to about this many MiB")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the (b, h) "
              "sequences are independent, so a multi-GPU run is B or H sharded with no "
              "communication and its throughput is N times the one-GPU figure.",
              file=sys.stderr)
        return 2

    import torch

    import gated_delta_rule_25_amd as g
    from gated_delta_rule_25_amd.inputs import WORKLOADS, make_inputs_torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    g.load()
    wl = WORKLOADS[args.workload]
    ins = make_inputs_torch(wl, device="cuda")
    torch.cuda.synchronize()
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.d_k, wl.d_v

    wall, kern_ms = time_prefill(g, ins, args.steps, args.warmup, args.impl, args.ring_mb)
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = sum(kern_ms) / len(kern_ms)
    head_tokens = B * T * H
    bytes_launch = prefill_bytes_per_head_token(dk, dv, T) * head_tokens
    flops_launch = prefill_flops_per_head_token(dk, dv) * head_tokens
    achieved_gbs = bytes_launch / (kern_avg * 1e-3) / 1e9
    tflops = flops_launch / (kern_avg * 1e-3) / 1e12
    print(f"[bench] prefill {args.impl}: {kern_avg:.3f} ms/launch (events), "
          f"{ms_per_step:.3f} ms/step (wall), {achieved_gbs:.0f} GB/s, {tflops:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    prologue = None
    if args.impl != "recurrent" and args.workload == "prefill_1p3b":
        # the same call with the fused prologue (q, k normalised and the gates taken from
        # pre-activations inside the kernels; the inputs serve as pre-activations)
        _, pk = time_prefill(g, ins, max(5, args.steps // 2), 1, args.impl, l2norm=True, gate_logits=True)
        pms = sum(pk) / len(pk)
        prologue = dict(kernel_ms=round(pms, 4), tokens_per_s=round(B * T / (pms * 1e-3), 1),
                        overhead_vs_plain=round(pms / kern_avg - 1.0, 4))
        print(f"[bench] prefill {args.impl} with the fused prologue: {pms:.3f} ms/launch "
              f"({100 * prologue['overhead_vs_plain']:+.1f}%)", file=sys.stderr, flush=True)

    cold_ms = time_prefill_cold(g, ins, 5, args.impl)
    print(f"[bench] prefill {args.impl} cold (512 MiB scrub between calls): {cold_ms:.3f} ms/launch",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(ins, args.cpu_heads)
        print(f"[bench] oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)
    del ins
    torch.cuda.empty_cache()

    others = {}
    bwd = None
    packed = None
    if not args.skip_others and args.workload == "prefill_1p3b" and args.impl != "recurrent":
        packed = varlen_leg(g, 10, kern_avg)
    if not args.skip_backward and args.workload == "prefill_1p3b":
        bwd = backward_leg(g, 5)
    norm = None
    if not args.skip_others and args.workload == "prefill_1p3b":
        norm = rmsnorm_leg(g, 20)
    sdm = None
    if not args.skip_others and args.workload == "prefill_1p3b":
        sdm = sdm_leg(g, 100)
    if not args.skip_others and args.workload == "prefill_1p3b" and args.impl != "recurrent":
        for name, steps in (("long_prefill", 3), ("gdn_scalar", 10), ("kda_scalar", 10)):
            others[name] = prefill_leg(g, name, steps, args.impl)
        if args.impl == "split":  # head size 256 and fp32 at d = 128 run on the two-kernel path only
            others["d256_prefill"] = prefill_leg(g, "d256_prefill", 10, args.impl)
            others["fp32_prefill"] = prefill_leg(g, "fp32_prefill", 5, args.impl)

    dec = {}
    decode_runs = () if args.skip_decode else ((256, args.decode_steps),
                                               (1024, max(1, args.decode_steps // 5)))
    for Bd, steps in decode_runs:
        dwall, dms = time_decode(g, Bd, 16, 128, steps, 10, seed=20254)
        davg = sum(dms) / len(dms)
        dbytes = decode_bytes_per_head(128, 128) * Bd * 16
        rate = dbytes / (davg * 1e-3) / 1e9
        # The 256 MiB state of B256 is partly served by the 256 MB Infinity Cache from one step to
        # the next, so its rate is an effective bandwidth (algorithmic bytes / time), not HBM
        # bandwidth. The 1 GiB state of B1024 cannot stay in that cache: its rate is the HBM figure.
        kind = "hbm" if Bd * 16 * 128 * 128 * 4 >= 1 << 30 else "effective (Infinity Cache assisted)"
        pre = "" if kind == "hbm" else "effective_"
        dec[f"B{Bd}"] = {"steps": steps, "kernel_ms": round(davg, 5),
                         "ms_per_step_wall": round(dwall * 1e3 / steps, 5), "bandwidth": kind,
                         pre + "gbs": round(rate, 1), pre + "frac": round(rate / HBM_PEAK_GBS, 4),
                         "head_state_updates_per_s": round(Bd * 16 / (davg * 1e-3), 1)}
        print(f"[bench] decode B={Bd}: {davg * 1e3:.1f} us/step, {rate:.1f} GB/s ({kind})",
              file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(1 << 28, device="cuda", dtype=torch.float32)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    digest = sources_digest(args.impl)
    rec = {
        "metric": "GDN-2 chunk fwd tokens/s (B8,H16,T4k,d128) + decode state HBM GB/s",
        "value": round(B * T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/f32" if args.impl == "recurrent" else "bf16-in/f16-mfma/f32-state",
        "data": "synthetic",
        "config": {"workload": f"GDN-2 layer prefill ({wl.name}) B{B} H{H} T{T} d_k=d_v={dk}, chunk 64",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv,
                   "impl": args.impl, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": (profiled_traffic(args.impl, digest)
                                 if args.workload == "prefill_1p3b" else None),
                     "sources": digest,
                     "kernels": KERNELS[args.impl],
                     "kernel_ms": round(kern_avg, 4),
                     "algorithmic_bytes": int(bytes_launch),
                     "mfma_frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        "cold_ms": round(cold_ms, 4),
        "other_prefill": others,
        "backward": bwd,
        "packed_prefill": packed,
        "output_rmsnorm": norm,
        "sparse_delta_memory": sdm,
        "prologue": prologue,
        "decode": dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
