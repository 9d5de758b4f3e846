// gdn2_api.cpp -- the C ABI declared in include/gdn2.h: argument checks, then launches.
//
// Every check runs on the host before anything is enqueued, so an argument error leaves the
// stream untouched. The library holds no state and allocates nothing.
#include "../../include/gdn2.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace {

bool dim_ok(int32_t d) { return d == 32 || d == 64 || d == 128; }
// The token-by-token kernel (decode, recurrent prefill) also takes 256.
bool dim_ok_tok(int32_t d) { return dim_ok(d) || d == 256; }

// Smallest workspace the two-kernel path accepts: the state buffer and one chunk slot.
size_t split_min_bytes(int32_t B, int32_t H, int32_t dk, int32_t dv, bool bf16) {
    return (size_t)B * H * dk * dv * 4 + gdn2::split_chunk_bytes(B, H, dk, bf16);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range_of(const void* p, uint64_t bytes) {
    Range r;
    if (p && bytes) {
        r.lo = reinterpret_cast<uintptr_t>(p);
        r.hi = r.lo + bytes;
    }
    return r;
}

bool overlap(const Range& a, const Range& b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// Element counts for the prefill layouts; false on overflow.
bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    if (a != 0 && b > (UINT64_MAX >> 2) / a) return false;
    *out = a * b;
    return true;
}

struct Sizes {
    uint64_t tok = 0;     // B*T*H
    uint64_t qk = 0;      // B*T*H*d_k elements
    uint64_t vw = 0;      // B*T*H*d_v elements
    uint64_t state = 0;   // B*H*d_k*d_v elements
    uint64_t scalar = 0;  // B*T*H elements (scalar gates)
};

bool sizes_of(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, Sizes* s) {
    uint64_t bt, bh;
    return mul_ok((uint64_t)B, (uint64_t)T, &bt) && mul_ok(bt, (uint64_t)H, &s->tok) &&
           mul_ok(s->tok, (uint64_t)dk, &s->qk) && mul_ok(s->tok, (uint64_t)dv, &s->vw) &&
           mul_ok((uint64_t)B, (uint64_t)H, &bh) && mul_ok(bh, (uint64_t)dk * (uint64_t)dv, &s->state) &&
           (s->scalar = s->tok, true) && s->qk < (1ull << 62) && s->vw < (1ull << 62);
}

// The chunked kernels launch one workgroup per (b, h, chunk) (the backward's key kernel four per
// chunk at d = 128); their grids, in threads, must stay below 2^31.
bool chunk_grids_ok(int32_t B, int32_t T, int32_t H, int32_t dk) {
    const long long nch = ((long long)T + 63) / 64;
    return (long long)B * H * (nch + 1) * (dk / 32) * 256 < (1ll << 31);
}

// Shared validation for prefill (T >= 0 tokens) and decode (T == 1, S0 == S_out == S).
gdn2_status validate(const void* q, const void* k, const void* v, const void* alpha,
                     const void* b, const void* w, const float* S0, const float* o,
                     const float* S_out, int32_t B, int32_t T, int32_t H, int32_t dk,
                     int32_t dv, gdn2_dtype dt, uint32_t flags, bool decode, bool tok = false) {
    if (dt != GDN2_BF16 && dt != GDN2_F32) return GDN2_ERR_UNSUPPORTED;
    if (flags & ~(uint32_t)(GDN2_ALPHA_SCALAR | GDN2_BETA_SCALAR | GDN2_QK_L2NORM | GDN2_GATE_LOGITS))
        return GDN2_ERR_UNSUPPORTED;
    if (B <= 0 || H <= 0 || T < 0) return GDN2_ERR_SHAPE;
    if (tok ? (!dim_ok_tok(dk) || !dim_ok_tok(dv)) : (!dim_ok(dk) || !dim_ok(dv))) return GDN2_ERR_UNSUPPORTED;
    Sizes sz;
    if (!sizes_of(B, T, H, dk, dv, &sz)) return GDN2_ERR_SHAPE;
    const bool bscalar = (flags & GDN2_BETA_SCALAR) != 0;
    const bool ascalar = (flags & GDN2_ALPHA_SCALAR) != 0;
    if (bscalar && w) return GDN2_ERR_UNSUPPORTED;  // w is implied by beta
    if (T > 0) {
        if (!q || !k || !v || !alpha || !b || !o || (!bscalar && !w)) return GDN2_ERR_NULL;
    }
    if (decode && (!S0 || !S_out)) return GDN2_ERR_NULL;
    const void* ptrs[] = {q, k, v, alpha, b, w, S0, o, S_out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_ALIGN;

    const uint64_t es = dt == GDN2_BF16 ? 2 : 4;
    const Range rq = range_of(q, sz.qk * es), rk = range_of(k, sz.qk * es);
    const Range rv = range_of(v, sz.vw * es);
    const Range ra = range_of(alpha, (ascalar ? sz.scalar : sz.qk) * es);
    const Range rb = range_of(b, (bscalar ? sz.scalar : sz.qk) * es);
    const Range rw = range_of(w, sz.vw * es);
    const Range rS0 = range_of(S0, sz.state * 4), rSo = range_of(S_out, sz.state * 4);
    const Range ro = range_of(o, sz.vw * 4);
    const Range ins[] = {rq, rk, rv, ra, rb, rw};
    for (const Range& r : ins) {
        if (overlap(ro, r) || overlap(rSo, r)) return GDN2_ERR_ALIAS;
        if (decode && overlap(rS0, r)) return GDN2_ERR_ALIAS;
    }
    if (overlap(ro, rS0) || overlap(ro, rSo)) return GDN2_ERR_ALIAS;
    if (overlap(rS0, rSo) && !(rS0.lo == rSo.lo && rS0.hi == rSo.hi)) return GDN2_ERR_ALIAS;
    return GDN2_OK;
}

gdn2_status run_recurrent(const void* q, const void* k, const void* v, const void* alpha,
                          const void* b, const void* w, const float* S0, float* o,
                          float* S_out, int32_t B, int32_t T, int32_t H, int32_t dk,
                          int32_t dv, gdn2_dtype dt, uint32_t flags, hipStream_t s) {
    if (!S_out && T == 0) return GDN2_OK;
    gdn2::RecurrentArgs a{q, k, v, alpha, b, w, S0, o, S_out, B, T, H, dk, dv,
                          dt == GDN2_BF16, flags};
    return gdn2::launch_recurrent(a, s) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

// The backward's checks and launch. cu == nullptr: B sequences of T tokens. Otherwise a packed
// batch: B sequences delimited by cu (device), T rows in all ([T, H, d] rows, [B, H, d_k, d_v]
// states).
gdn2_status run_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                    const void* w, const float* S0, const float* dO, const float* dS_T, float* dq,
                    float* dk, float* dv, float* dalpha, float* db, float* dw, float* dS0,
                    const int32_t* cu, int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                    gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                    size_t workspace_bytes, void* stream, bool saved = false) {
    if (in_dtype != GDN2_BF16 ||
        (gate_flags & ~(uint32_t)(GDN2_ALPHA_SCALAR | GDN2_BETA_SCALAR | GDN2_QK_L2NORM | GDN2_GATE_LOGITS)) != 0u)
        return GDN2_ERR_UNSUPPORTED;
    const bool as = (gate_flags & GDN2_ALPHA_SCALAR) != 0, bs = (gate_flags & GDN2_BETA_SCALAR) != 0;
    if (bs && (w || dw)) return GDN2_ERR_UNSUPPORTED;  // w is implied by beta; dbeta goes to db
    if (B <= 0 || H <= 0 || T < 0) return GDN2_ERR_SHAPE;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return GDN2_ERR_UNSUPPORTED;
    const int32_t Brow = cu ? 1 : B;  // sequences along the row axis
    Sizes sz, st;
    if (!sizes_of(Brow, T, H, d_k, d_v, &sz) || !sizes_of(B, 1, H, d_k, d_v, &st)) return GDN2_ERR_SHAPE;
    if (cu ? gdn2::varlen_chunk_bound(B, T) * H * (d_k / 32) * 256 >= (1l << 31) : !chunk_grids_ok(B, T, H, d_k))
        return GDN2_ERR_SHAPE;
    if (!gdn2::bwd_supported(T, H, d_k, d_v, true, gate_flags)) return GDN2_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !alpha || !b || (!bs && !w) || !dO || !dq || !dk || !dv || !dalpha || !db ||
                  (!bs && !dw)))
        return GDN2_ERR_NULL;
    const void* ptrs[] = {q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_ALIGN;
    size_t need = 0;
    if (T > 0) {
        need = cu ? gdn2::bwd_varlen_workspace_bytes(B, T, H, d_k, d_v, gate_flags)
                  : gdn2::bwd_workspace_bytes(B, T, H, d_k, d_v, gate_flags);
        if (!workspace || workspace_bytes < need) return GDN2_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
    }
    const uint64_t na = as ? sz.scalar : sz.qk, nb = bs ? sz.scalar : sz.qk;  // alpha, b elements
    const Range ins[] = {range_of(q, sz.qk * 2), range_of(k, sz.qk * 2), range_of(v, sz.vw * 2),
                         range_of(alpha, na * 2), range_of(b, nb * 2), range_of(w, sz.vw * 2),
                         range_of(S0, st.state * 4), range_of(dO, sz.vw * 4), range_of(dS_T, st.state * 4),
                         range_of(cu, cu ? ((uint64_t)B + 1) * 4 : 0)};
    const Range outs[] = {range_of(dq, sz.qk * 4), range_of(dk, sz.qk * 4), range_of(dalpha, na * 4),
                          range_of(db, nb * 4), range_of(dv, sz.vw * 4), range_of(dw, sz.vw * 4),
                          range_of(dS0, st.state * 4), range_of(T > 0 ? workspace : nullptr, need)};
    const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
    for (int i = 0; i < nout; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return GDN2_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return GDN2_ERR_ALIAS;
    }
    gdn2::BwdArgs a{q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0,
                    B, T, H, d_k, d_v, true, gate_flags, workspace, workspace_bytes};
    a.cu_seqlens = cu;
    a.saved = saved;
    const hipError_t e = gdn2::launch_bwd(a, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return GDN2_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

// The checks and launch of gdn2_rmsnorm_bwd. With fixed_scratch, the dweight partials go to the
// library's own device array (no workspace argument, nothing allocated).
gdn2_status rmsnorm_bwd_checked(const float* x, const float* weight, const float* dy, float* dx, float* dweight,
                                int64_t rows, int32_t d, float eps, void* workspace, size_t workspace_bytes,
                                bool fixed_scratch, void* stream) {
    if (rows < 0 || (uint64_t)rows > (1ull << 40)) return GDN2_ERR_SHAPE;
    if (!dim_ok_tok(d) || !(eps >= 0.f && eps <= 3.0e38f)) return GDN2_ERR_UNSUPPORTED;
    if (rows > 0 && (!x || !dy || !dx)) return GDN2_ERR_NULL;
    const void* ptrs[] = {x, weight, dy, dx, dweight};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_ALIGN;
    const size_t need = dweight ? gdn2::rmsnorm_bwd_workspace_bytes((long)rows, d) : 0;
    if (fixed_scratch) {
        workspace = nullptr;  // looked up below, after every argument check
    } else if (need > 0) {
        if (!workspace || workspace_bytes < need) return GDN2_ERR_WORKSPACE;
        if (!aligned16(workspace)) return GDN2_ERR_ALIGN;
    }
    if (rows == 0 && !dweight) return GDN2_OK;
    const uint64_t n = (uint64_t)rows * (uint64_t)d;
    const Range rx = range_of(x, n * 4), rwt = range_of(weight, (uint64_t)d * 4), rdy = range_of(dy, n * 4),
                rdx = range_of(dx, n * 4), rdw = range_of(dweight, (uint64_t)d * 4),
                rws = range_of(need && !fixed_scratch ? workspace : nullptr, need);
    // dx may be dy itself (each lane reads its dy before it writes the same elements of dx)
    if (overlap(rdx, rx) || overlap(rdx, rwt) || (overlap(rdx, rdy) && dx != dy) || overlap(rdx, rdw) ||
        overlap(rdx, rws))
        return GDN2_ERR_ALIAS;
    if (overlap(rdw, rx) || overlap(rdw, rwt) || overlap(rdw, rdy) || overlap(rdw, rws)) return GDN2_ERR_ALIAS;
    if (overlap(rws, rx) || overlap(rws, rwt) || overlap(rws, rdy)) return GDN2_ERR_ALIAS;
    if (fixed_scratch && need > 0) {  // the library's own array on the current device
        size_t have = 0;
        if (gdn2::rmsnorm_scratch(&workspace, &have) != hipSuccess) return GDN2_ERR_HIP;
        if (need > have) return GDN2_ERR_SCRATCH;
    }
    gdn2::RmsNormArgs a{x, weight, nullptr, false, dy, dx, dweight, workspace, (long)rows, d, eps};
    const hipError_t e = gdn2::launch_rmsnorm_bwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

// The checks and launch of gdn2_chunk_fwd_varlen, and with `save` of gdn2_chunk_fwd_varlen_save
// (the workspace is then the backward's, which keeps what gdn2_chunk_bwd_varlen_saved reads).
gdn2_status varlen_fwd(const void* q, const void* k, const void* v, const void* alpha, const void* b, const void* w,
                       const float* S0, float* o, float* S_out, const int32_t* cu_seqlens, int32_t N, int32_t T_total,
                       int32_t H, int32_t d_k, int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                       size_t workspace_bytes, void* stream, bool save) {
    if (N <= 0) return GDN2_ERR_SHAPE;
    // the token rows are one sequence of T_total tokens as far as sizes go; the states separately
    gdn2_status st = validate(q, k, v, alpha, b, w, nullptr, o, nullptr, 1, T_total, H, d_k, d_v,
                              in_dtype, gate_flags, false);
    if (st != GDN2_OK) return st;
    if (!cu_seqlens) return GDN2_ERR_NULL;
    const bool bf16 = in_dtype == GDN2_BF16;
    if (save && (!bf16 || !gdn2::bwd_supported(T_total, H, d_k, d_v, true, gate_flags))) return GDN2_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return GDN2_ERR_ALIGN;
    if ((S0 && !aligned16(S0)) || (S_out && !aligned16(S_out))) return GDN2_ERR_ALIGN;
    if (save && T_total == 0)  // no rows: nothing to save; S_out <- S0 (or zeros) per sequence
        return run_recurrent(q, k, v, alpha, b, w, S0, o, S_out, N, 0, H, d_k, d_v, in_dtype, gate_flags,
                             static_cast<hipStream_t>(stream));
    if (!workspace) return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
    if (!gdn2::varlen_fwd_supported(T_total, H, d_k, d_v, bf16)) return GDN2_ERR_UNSUPPORTED;
    // one workgroup per (chunk bound, head) in prep and per (sequence, head, value tile) in the
    // chain: both grids (in threads) must stay below 2^31
    if (gdn2::varlen_chunk_bound(N, T_total) * H * 256 >= (1l << 31)) return GDN2_ERR_SHAPE;
    if (((long)N * H + 7) / 8 * 8 * (d_v / (d_k < 64 ? d_k : 64)) * 512 >= (1l << 31)) return GDN2_ERR_SHAPE;
    Sizes sz, states;
    if (!sizes_of(1, T_total, H, d_k, d_v, &sz) || !sizes_of(N, 1, H, d_k, d_v, &states)) return GDN2_ERR_SHAPE;
    const size_t need = save ? gdn2::bwd_varlen_workspace_bytes(N, T_total, H, d_k, d_v, gate_flags)
                             : gdn2::varlen_workspace_bytes(N, T_total, H, d_k, d_v, bf16);
    if (workspace_bytes < need) return GDN2_ERR_WORKSPACE;
    const uint64_t es = bf16 ? 2 : 4;
    const bool as = (gate_flags & GDN2_ALPHA_SCALAR) != 0, bs = (gate_flags & GDN2_BETA_SCALAR) != 0;
    const Range ins[] = {range_of(q, sz.qk * es), range_of(k, sz.qk * es), range_of(v, sz.vw * es),
                         range_of(alpha, (as ? sz.scalar : sz.qk) * es), range_of(b, (bs ? sz.scalar : sz.qk) * es),
                         range_of(w, sz.vw * es), range_of(cu_seqlens, ((uint64_t)N + 1) * 4)};
    const Range rS0 = range_of(S0, states.state * 4), rSo = range_of(S_out, states.state * 4);
    const Range ro = range_of(o, sz.vw * 4), rws = range_of(workspace, save ? need : workspace_bytes);
    for (const Range& r : ins)
        if (overlap(rSo, r) || overlap(ro, r) || overlap(rws, r)) return GDN2_ERR_ALIAS;
    if (overlap(ro, rS0) || overlap(ro, rSo) || overlap(rws, rS0) || overlap(rws, rSo) || overlap(rws, ro))
        return GDN2_ERR_ALIAS;
    if (overlap(rS0, rSo) && !(rS0.lo == rSo.lo && rS0.hi == rSo.hi)) return GDN2_ERR_ALIAS;
    gdn2::ChunkArgs a{q, k, v, alpha, b, w, S0, o, S_out, N, T_total, H, d_k, d_v, bf16, gate_flags,
                      workspace, workspace_bytes};
    a.cu_seqlens = cu_seqlens;
    const hipError_t e = save ? gdn2::launch_fwd_save(a, static_cast<hipStream_t>(stream))
                              : gdn2::launch_split_varlen(a, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return GDN2_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

}  // namespace

extern "C" {

gdn2_status gdn2_recurrent_fwd(const void* q, const void* k, const void* v, const void* alpha,
                               const void* b, const void* w, const float* S0, float* o,
                               float* S_out, int32_t B, int32_t T, int32_t H, int32_t d_k,
                               int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                               void* stream) {
    const gdn2_status st = validate(q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v,
                                    in_dtype, gate_flags, false, true);
    if (st != GDN2_OK) return st;
    return run_recurrent(q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, in_dtype,
                         gate_flags, static_cast<hipStream_t>(stream));
}

size_t gdn2_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                      int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags) {
    if (B <= 0 || H <= 0 || T <= 0 || !dim_ok_tok(d_k) || !dim_ok_tok(d_v)) return 0;
    const bool bf16 = in_dtype == GDN2_BF16;
    if (!gdn2::split_fwd_supported(T, H, d_k, d_v, bf16)) return 0;
    return gdn2::split_workspace_bytes(B, T, H, d_k, d_v, bf16);
}

gdn2_status gdn2_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                           const void* b, const void* w, const float* S0, float* o,
                           float* S_out, int32_t B, int32_t T, int32_t H, int32_t d_k,
                           int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
    // head size 256 passes here and is taken by the two-kernel path only (bf16, with a workspace)
    gdn2_status st = validate(q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, in_dtype,
                              gate_flags, false, true);
    if (st != GDN2_OK) return st;
    if (!chunk_grids_ok(B, T, H, d_k)) return GDN2_ERR_SHAPE;
    const bool bf16 = in_dtype == GDN2_BF16;
    const bool fused = gdn2::fused_supported(T, H, d_k, d_v, bf16);
    const bool split = workspace && workspace_bytes > 0 && gdn2::split_fwd_supported(T, H, d_k, d_v, bf16);
    if (split) {
        const size_t min_bytes = split_min_bytes(B, H, d_k, d_v, bf16);
        if (workspace_bytes < min_bytes) return GDN2_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
        const Range rws = range_of(workspace, workspace_bytes);
        const uint64_t es = bf16 ? 2 : 4;
        Sizes sz;
        sizes_of(B, T, H, d_k, d_v, &sz);
        const Range others[] = {range_of(q, sz.qk * es), range_of(k, sz.qk * es), range_of(v, sz.vw * es),
                                range_of(alpha, ((gate_flags & GDN2_ALPHA_SCALAR) ? sz.scalar : sz.qk) * es),
                                range_of(b, ((gate_flags & GDN2_BETA_SCALAR) ? sz.scalar : sz.qk) * es),
                                range_of(w, sz.vw * es),
                                range_of(S0, sz.state * 4), range_of(o, sz.vw * 4), range_of(S_out, sz.state * 4)};
        for (const Range& r : others)
            if (overlap(rws, r)) return GDN2_ERR_ALIAS;
    } else if (!fused && (!gdn2::chunk_supported(T, H, d_k, d_v, bf16) ||
                          (gate_flags & (GDN2_QK_L2NORM | GDN2_GATE_LOGITS)))) {  // no prologue on the single kernel
        return GDN2_ERR_UNSUPPORTED;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {  // nothing to chunk: S_out <- S0 (or zeros)
        return run_recurrent(q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, in_dtype,
                             gate_flags, s);
    }
    gdn2::ChunkArgs a{q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, bf16, gate_flags,
                      split ? workspace : nullptr, split ? workspace_bytes : 0};
    const hipError_t e = split ? gdn2::launch_split(a, s) : fused ? gdn2::launch_fused(a, s) : gdn2::launch_chunk(a, s);
    if (e == hipErrorNotSupported) return GDN2_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

size_t gdn2_chunk_fwd_varlen_workspace_bytes(int32_t N, int32_t T_total, int32_t H, int32_t d_k,
                                             int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags) {
    if (N <= 0 || H <= 0 || T_total < 0 || !dim_ok(d_k) || !dim_ok(d_v)) return 0;
    const bool bf16 = in_dtype == GDN2_BF16;
    if (!gdn2::varlen_fwd_supported(T_total, H, d_k, d_v, bf16)) return 0;
    return gdn2::varlen_workspace_bytes(N, T_total, H, d_k, d_v, bf16);
}

gdn2_status gdn2_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* alpha,
                                  const void* b, const void* w, const float* S0, float* o,
                                  float* S_out, const int32_t* cu_seqlens, int32_t N,
                                  int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                  gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return varlen_fwd(q, k, v, alpha, b, w, S0, o, S_out, cu_seqlens, N, T_total, H, d_k, d_v, in_dtype, gate_flags,
                      workspace, workspace_bytes, stream, false);
}

gdn2_status gdn2_chunk_fwd_varlen_save(const void* q, const void* k, const void* v, const void* alpha,
                                       const void* b, const void* w, const float* S0, float* o,
                                       float* S_out, const int32_t* cu_seqlens, int32_t N,
                                       int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                       gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    return varlen_fwd(q, k, v, alpha, b, w, S0, o, S_out, cu_seqlens, N, T_total, H, d_k, d_v, in_dtype, gate_flags,
                      workspace, workspace_bytes, stream, true);
}

gdn2_status gdn2_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                             const void* b, const void* w, float* S, float* o, int32_t B,
                             int32_t H, int32_t d_k, int32_t d_v, gdn2_dtype in_dtype,
                             uint32_t gate_flags, void* stream) {
    // A [B, H, d] input is a [B, 1, H, d] input: the decode step is one token of prefill.
    const gdn2_status st = validate(q, k, v, alpha, b, w, S, o, S, B, 1, H, d_k, d_v, in_dtype,
                                    gate_flags, true, true);
    if (st != GDN2_OK) return st;
    return run_recurrent(q, k, v, alpha, b, w, S, o, S, B, 1, H, d_k, d_v, in_dtype,
                         gate_flags, static_cast<hipStream_t>(stream));
}

gdn2_status gdn2_decode_step_slots(const void* q, const void* k, const void* v, const void* alpha,
                                   const void* b, const void* w, float* S_pool, const int32_t* slots,
                                   float* o, int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                                   int32_t n_slots, gdn2_dtype in_dtype, uint32_t gate_flags,
                                   void* stream) {
    if (n_slots <= 0) return GDN2_ERR_SHAPE;
    // the inputs and o are [B, H, d] (checked as one token of B sequences); the pool separately
    gdn2_status st = validate(q, k, v, alpha, b, w, nullptr, o, nullptr, B, 1, H, d_k, d_v, in_dtype,
                              gate_flags, false, true);
    if (st != GDN2_OK) return st;
    if (!slots || !S_pool) return GDN2_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(slots) & 3u) != 0 || !aligned16(S_pool)) return GDN2_ERR_ALIGN;
    Sizes sz, pool;
    if (!sizes_of(B, 1, H, d_k, d_v, &sz) || !sizes_of(n_slots, 1, H, d_k, d_v, &pool)) return GDN2_ERR_SHAPE;
    const uint64_t es = in_dtype == GDN2_BF16 ? 2 : 4;
    const bool as = (gate_flags & GDN2_ALPHA_SCALAR) != 0, bs = (gate_flags & GDN2_BETA_SCALAR) != 0;
    const Range rp = range_of(S_pool, pool.state * 4), ro = range_of(o, sz.vw * 4);
    const Range ins[] = {range_of(q, sz.qk * es), range_of(k, sz.qk * es), range_of(v, sz.vw * es),
                         range_of(alpha, (as ? sz.scalar : sz.qk) * es), range_of(b, (bs ? sz.scalar : sz.qk) * es),
                         range_of(w, sz.vw * es), range_of(slots, (uint64_t)B * 4)};
    for (const Range& r : ins)
        if (overlap(rp, r) || overlap(ro, r)) return GDN2_ERR_ALIAS;
    if (overlap(rp, ro)) return GDN2_ERR_ALIAS;
    gdn2::RecurrentArgs a{q, k, v, alpha, b, w, S_pool, o, S_pool, B, 1, H, d_k, d_v,
                          in_dtype == GDN2_BF16, gate_flags};
    a.slots = slots;
    a.n_slots = n_slots;
    return gdn2::launch_recurrent(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

size_t gdn2_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                      gdn2_dtype in_dtype, uint32_t gate_flags) {
    if (B <= 0 || H <= 0 || T <= 0 || !dim_ok(d_k) || !dim_ok(d_v)) return 0;
    if (!gdn2::bwd_supported(T, H, d_k, d_v, in_dtype == GDN2_BF16, gate_flags)) return 0;
    Sizes sz;
    if (!sizes_of(B, T, H, d_k, d_v, &sz)) return 0;
    return gdn2::bwd_workspace_bytes(B, T, H, d_k, d_v, gate_flags);
}

gdn2_status gdn2_chunk_bwd(const void* q, const void* k, const void* v, const void* alpha,
                           const void* b, const void* w, const float* S0, const float* dO,
                           const float* dS_T, float* dq, float* dk, float* dv, float* dalpha,
                           float* db, float* dw, float* dS0, int32_t B, int32_t T, int32_t H,
                           int32_t d_k, int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return run_bwd(q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0, nullptr, B, T, H, d_k, d_v,
                   in_dtype, gate_flags, workspace, workspace_bytes, stream);
}

gdn2_status gdn2_chunk_fwd_save(const void* q, const void* k, const void* v, const void* alpha,
                                const void* b, const void* w, const float* S0, float* o, float* S_out,
                                int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                                size_t workspace_bytes, void* stream) {
    gdn2_status st = validate(q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, in_dtype, gate_flags, false);
    if (st != GDN2_OK) return st;
    if (in_dtype != GDN2_BF16 || !gdn2::bwd_supported(T, H, d_k, d_v, true, gate_flags)) return GDN2_ERR_UNSUPPORTED;
    if (!chunk_grids_ok(B, T, H, d_k)) return GDN2_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)  // nothing to save: S_out <- S0 (or zeros)
        return run_recurrent(q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, in_dtype, gate_flags, s);
    const size_t need = gdn2::bwd_workspace_bytes(B, T, H, d_k, d_v, gate_flags);
    if (!workspace || workspace_bytes < need) return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
    Sizes sz;
    sizes_of(B, T, H, d_k, d_v, &sz);
    const Range rws = range_of(workspace, need);
    const Range others[] = {range_of(q, sz.qk * 2), range_of(k, sz.qk * 2), range_of(v, sz.vw * 2),
                            range_of(alpha, ((gate_flags & GDN2_ALPHA_SCALAR) ? sz.scalar : sz.qk) * 2),
                            range_of(b, ((gate_flags & GDN2_BETA_SCALAR) ? sz.scalar : sz.qk) * 2),
                            range_of(w, sz.vw * 2), range_of(S0, sz.state * 4), range_of(o, sz.vw * 4),
                            range_of(S_out, sz.state * 4)};
    for (const Range& r : others)
        if (overlap(rws, r)) return GDN2_ERR_ALIAS;
    gdn2::ChunkArgs a{q, k, v, alpha, b, w, S0, o, S_out, B, T, H, d_k, d_v, true, gate_flags, workspace,
                      workspace_bytes};
    const hipError_t e = gdn2::launch_fwd_save(a, s);
    if (e == hipErrorNotSupported) return GDN2_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status gdn2_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* alpha,
                                 const void* b, const void* w, const float* S0, const float* dO,
                                 const float* dS_T, float* dq, float* dk, float* dv, float* dalpha,
                                 float* db, float* dw, float* dS0, int32_t B, int32_t T, int32_t H,
                                 int32_t d_k, int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return run_bwd(q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0, nullptr, B, T, H, d_k, d_v,
                   in_dtype, gate_flags, workspace, workspace_bytes, stream, true);
}

gdn2_status gdn2_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* alpha,
                                  const void* b, const void* w, const float* S0, const float* dO,
                                  const float* dS_T, float* dq, float* dk, float* dv, float* dalpha,
                                  float* db, float* dw, float* dS0, const int32_t* cu_seqlens, int32_t N,
                                  int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                  gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (!cu_seqlens) return GDN2_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return GDN2_ERR_ALIGN;
    return run_bwd(q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0, cu_seqlens, N, T_total, H,
                   d_k, d_v, in_dtype, gate_flags, workspace, workspace_bytes, stream);
}

gdn2_status gdn2_chunk_bwd_varlen_saved(const void* q, const void* k, const void* v, const void* alpha,
                                        const void* b, const void* w, const float* S0, const float* dO,
                                        const float* dS_T, float* dq, float* dk, float* dv, float* dalpha,
                                        float* db, float* dw, float* dS0, const int32_t* cu_seqlens, int32_t N,
                                        int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                        gdn2_dtype in_dtype, uint32_t gate_flags, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (!cu_seqlens) return GDN2_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return GDN2_ERR_ALIGN;
    return run_bwd(q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0, cu_seqlens, N, T_total, H,
                   d_k, d_v, in_dtype, gate_flags, workspace, workspace_bytes, stream, true);
}

size_t gdn2_chunk_bwd_varlen_workspace_bytes(int32_t N, int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                             gdn2_dtype in_dtype, uint32_t gate_flags) {
    if (N <= 0 || H <= 0 || T_total <= 0 || !dim_ok(d_k) || !dim_ok(d_v)) return 0;
    if (!gdn2::bwd_supported(T_total, H, d_k, d_v, in_dtype == GDN2_BF16, gate_flags)) return 0;
    Sizes sz;
    if (!sizes_of(1, T_total, H, d_k, d_v, &sz)) return 0;
    return gdn2::bwd_varlen_workspace_bytes(N, T_total, H, d_k, d_v, gate_flags);
}

gdn2_status gdn2_rmsnorm_fwd(const float* x, const float* weight, void* y, int64_t rows, int32_t d, float eps,
                             gdn2_dtype y_dtype, void* stream) {
    if (rows < 0) return GDN2_ERR_SHAPE;
    if (!dim_ok_tok(d) || (y_dtype != GDN2_BF16 && y_dtype != GDN2_F32) || !(eps >= 0.f && eps <= 3.0e38f))
        return GDN2_ERR_UNSUPPORTED;
    if (rows == 0) return GDN2_OK;
    if (!x || !y) return GDN2_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || (weight && !aligned16(weight))) return GDN2_ERR_ALIGN;
    const uint64_t n = (uint64_t)rows * (uint64_t)d;
    if ((uint64_t)rows > (1ull << 40) || (n + 1023) / 1024 * 256 >= (1ull << 31)) return GDN2_ERR_SHAPE;  // grid threads
    const bool bf = y_dtype == GDN2_BF16;
    const Range rx = range_of(x, n * 4), ry = range_of(y, n * (bf ? 2 : 4)), rw = range_of(weight, (uint64_t)d * 4);
    if (overlap(ry, rw) || (overlap(ry, rx) && !(y == x && !bf))) return GDN2_ERR_ALIAS;
    gdn2::RmsNormArgs a{x, weight, y, bf, nullptr, nullptr, nullptr, nullptr, (long)rows, d, eps};
    const hipError_t e = gdn2::launch_rmsnorm_fwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

size_t gdn2_rmsnorm_bwd_workspace_bytes(int64_t rows, int32_t d) {
    if (rows < 0 || (uint64_t)rows > (1ull << 40) || !dim_ok_tok(d)) return 0;
    return gdn2::rmsnorm_bwd_workspace_bytes((long)rows, d);
}

gdn2_status gdn2_rmsnorm_bwd(const float* x, const float* weight, const float* dy, float* dx, float* dweight,
                             int64_t rows, int32_t d, float eps, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return rmsnorm_bwd_checked(x, weight, dy, dx, dweight, rows, d, eps, workspace, workspace_bytes, false, stream);
}

gdn2_status gdn2_rmsnorm_bwd_noalloc(const float* x, const float* weight, const float* dy, float* dx,
                                     float* dweight, int64_t rows, int32_t d, float eps, void* stream) {
    return rmsnorm_bwd_checked(x, weight, dy, dx, dweight, rows, d, eps, nullptr, 0, true, stream);
}

const char* gdn2_status_str(gdn2_status s) {
    switch (s) {
        case GDN2_OK: return "ok";
        case GDN2_ERR_NULL: return "a required pointer is NULL";
        case GDN2_ERR_SHAPE: return "invalid shape";
        case GDN2_ERR_UNSUPPORTED: return "unsupported head size, dtype or flags";
        case GDN2_ERR_ALIGN: return "pointer not 16-byte aligned";
        case GDN2_ERR_ALIAS: return "an output overlaps an input";
        case GDN2_ERR_HIP: return "HIP launch error";
        case GDN2_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN2_ERR_SCRATCH: return "size beyond the library's fixed scratch";
    }
    return "unknown status";
}

gdn2_status gdn2_sdm_address(const void* x, const void* C1, const void* C2, int64_t rows, int32_t H, int32_t d_k,
                             int32_t n, int32_t m, gdn2_dtype dtype, int32_t* idx, float* weight, void* stream) {
    if (rows < 0 || H <= 0) return GDN2_ERR_SHAPE;
    if ((dtype != GDN2_BF16 && dtype != GDN2_F32) || !gdn2::sdm_address_supported(d_k, n, m))
        return GDN2_ERR_UNSUPPORTED;
    if (!C1 || !C2) return GDN2_ERR_NULL;
    if (rows > 0 && (!x || !idx || !weight)) return GDN2_ERR_NULL;
    if (!aligned16(C1) || !aligned16(C2) || (x && !aligned16(x)) || (idx && !aligned16(idx)) ||
        (weight && !aligned16(weight)))
        return GDN2_ERR_ALIGN;
    uint64_t queries, xs;
    if (!mul_ok((uint64_t)rows, (uint64_t)H, &queries) || !mul_ok(queries, (uint64_t)d_k, &xs) ||
        queries > (1ull << 40))
        return GDN2_ERR_SHAPE;
    if (rows == 0) return GDN2_OK;
    const uint64_t es = dtype == GDN2_BF16 ? 2 : 4;
    const uint64_t table = (uint64_t)H * n * (d_k / 2) * es;
    const Range ins[] = {range_of(x, xs * es), range_of(C1, table), range_of(C2, table)};
    const Range ri = range_of(idx, queries * m * 4), rw = range_of(weight, queries * m * 4);
    for (const Range& r : ins)
        if (overlap(ri, r) || overlap(rw, r)) return GDN2_ERR_ALIAS;
    if (overlap(ri, rw)) return GDN2_ERR_ALIAS;
    gdn2::SdmAddressArgs a{x, C1, C2, (long)queries, H, d_k, n, m, dtype == GDN2_BF16, idx, weight};
    return gdn2::launch_sdm_address(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status gdn2_sdm_fwd(const void* v, const void* alpha, const void* b, const void* w, const int32_t* widx,
                         const float* wwt, const int32_t* ridx, const float* rwt, float* M, double* stamp,
                         double* L, float* o, int32_t B, int32_t T, int32_t H, int64_t N, int32_t d_v, int32_t W,
                         int32_t R, gdn2_dtype dtype, void* stream) {
    if (B < 0 || T < 0 || H <= 0 || N <= 0 || N > 0x7fffffff) return GDN2_ERR_SHAPE;
    if ((dtype != GDN2_BF16 && dtype != GDN2_F32) || !gdn2::sdm_fwd_supported(d_v, W, R)) return GDN2_ERR_UNSUPPORTED;
    if (W > N || R > N) return GDN2_ERR_SHAPE;
    if (B == 0) return GDN2_OK;
    if (!M || !stamp || !L) return GDN2_ERR_NULL;
    if (T > 0 && (!v || !alpha || !b || !widx || !wwt || !ridx || !rwt || !o)) return GDN2_ERR_NULL;
    const void* ptrs[] = {v, alpha, b, w, widx, wwt, ridx, rwt, M, stamp, L, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_ALIGN;
    uint64_t bh, tok, mem, vw, bookkeeping;
    const uint64_t tiles = (uint64_t)(d_v / 64);
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || !mul_ok(bh, (uint64_t)T, &tok) ||
        !mul_ok(bh, (uint64_t)N, &mem) || !mul_ok(mem, (uint64_t)d_v, &mem) || !mul_ok(tok, (uint64_t)d_v, &vw) ||
        !mul_ok(bh * tiles, (uint64_t)N, &bookkeeping) || bh * tiles >= (1ull << 31))
        return GDN2_ERR_SHAPE;
    if (T == 0) return GDN2_OK;
    const uint64_t es = dtype == GDN2_BF16 ? 2 : 4;
    const Range ins[] = {range_of(v, vw * es), range_of(alpha, tok * es), range_of(b, tok * es), range_of(w, vw * es),
                         range_of(widx, tok * W * 4), range_of(wwt, tok * W * 4), range_of(ridx, tok * R * 4),
                         range_of(rwt, tok * R * 4)};
    const Range outs[] = {range_of(M, mem * 4), range_of(stamp, bookkeeping * 8), range_of(L, bh * tiles * 8),
                          range_of(o, vw * 4)};
    const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
    for (int i = 0; i < nout; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return GDN2_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return GDN2_ERR_ALIAS;
    }
    gdn2::SdmFwdArgs a{v, alpha, b, w, widx, wwt, ridx, rwt, M, stamp, L, o, B, T, H, (long)N, d_v, W, R,
                       dtype == GDN2_BF16};
    return gdn2::launch_sdm_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status gdn2_sdm_fold(float* M, double* stamp, double* L, int32_t B, int32_t H, int64_t N, int32_t d_v,
                          void* stream) {
    if (B < 0 || H <= 0 || N <= 0 || N > 0x7fffffff) return GDN2_ERR_SHAPE;
    if (d_v != 64 && d_v != 128 && d_v != 256) return GDN2_ERR_UNSUPPORTED;
    if (B == 0) return GDN2_OK;
    if (!M || !stamp || !L) return GDN2_ERR_NULL;
    if (!aligned16(M) || !aligned16(stamp) || !aligned16(L)) return GDN2_ERR_ALIGN;
    uint64_t bh, mem, bookkeeping;
    const uint64_t tiles = (uint64_t)(d_v / 64);
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || !mul_ok(bh, (uint64_t)N, &mem) || !mul_ok(mem, (uint64_t)d_v, &mem) ||
        !mul_ok(bh * tiles, (uint64_t)N, &bookkeeping) || bh * tiles * 64 >= (1ull << 31))
        return GDN2_ERR_SHAPE;
    const Range rM = range_of(M, mem * 4), rS = range_of(stamp, bookkeeping * 8), rL = range_of(L, bh * tiles * 8);
    if (overlap(rM, rS) || overlap(rM, rL) || overlap(rS, rL)) return GDN2_ERR_ALIAS;
    return gdn2::launch_sdm_fold(M, stamp, L, (long)bh, (long)N, d_v, static_cast<hipStream_t>(stream)) == hipSuccess
               ? GDN2_OK
               : GDN2_ERR_HIP;
}

int gdn2_abi_version(void) { return GDN2_ABI_VERSION; }

}  // extern "C"
