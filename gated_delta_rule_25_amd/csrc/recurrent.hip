// recurrent.hip -- token-by-token Gated DeltaNet-2 recurrence on gfx950 (fp32 arithmetic).
//
// Update [page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph
// "Техническая схема", state-update equation]:
//     S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T,  o_t = S_t^T q_t.
// Written per value column c, with the decay folded into the two reads of the old state:
//     r_c     = sum_i alpha_i b_i k_i S_ic            (erase read of the decayed state)
//     delta_c = w_c v_c - r_c
//     S'_ic   = alpha_i S_ic + k_i delta_c
//     o_c     = sum_i alpha_i q_i S_ic + (q . k) delta_c      (= sum_i q_i S'_ic)
// so each state element is read and written once per token.
//
// Work split: one wavefront owns a 32-column slice of one (b, h) state, d_k x 32 fp32 held in
// VGPRs for the whole sequence. Lane = 8*rg + cq: it holds rows rg*R .. rg*R+R-1 (R = d_k/8)
// and columns 4*cq .. 4*cq+3 of the slice. The two column reductions over d_k are butterflies
// across the 8 row groups (lane xor 8, 16, 32), so a token needs no LDS and no barrier.
// The decode step is this kernel with T = 1 and S0 == S_out == S.
//
// Prologue (PRO): bit 0, q and k are L2-normalised over d_k per token (their sums of squares
// ride in the same butterflies, and the reductions are scaled afterwards: r by 1/|k|, the readout
// by 1/|q|, q.k by both); bit 1, alpha, b and w arrive as pre-activations and go through the
// logistic sigmoid when loaded [same page, paragraph "Архитектурно": L2-normalised q/k,
// sigmoid gates].
#include "common.h"
#include "kernels.h"

namespace gdn2 {

namespace {

__device__ __forceinline__ float sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));  // rcp within 1 ulp
}

// ONE: exactly one token (the decode step): no next-token prefetch, so fewer registers and more
// wavefronts per SIMD (which helps while the state sits in the Infinity Cache; streaming it from
// HBM, the general kernel is faster).
template <int DK, bool BF16, bool ASCALAR, bool BSCALAR, int PRO, bool ONE>
__global__ void __launch_bounds__(256)
recurrent_kernel(const void* __restrict__ q, const void* __restrict__ k,
                 const void* __restrict__ v, const void* __restrict__ alpha,
                 const void* __restrict__ b, const void* __restrict__ w,
                 const float* S0, float* __restrict__ o, float* S_out, int B, int T, int H,
                 int DV, const int* __restrict__ slots, int n_slots) {
    constexpr int R = DK / 8;  // rows per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int item = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    const int tiles = DV / 32;
    if (item >= B * H * tiles) return;  // whole wave exits together
    const int tile = item % tiles;
    const int bh = item / tiles;
    const int hh = bh % H;
    const int bb = bh / H;
    const int rg = lane >> 3, cq = lane & 7;
    const int row0 = rg * R;
    const int col0 = tile * 32 + cq * 4;

    // the state of batch row bb: its own, or pool entry slots[bb] (rows whose slot lies outside
    // the pool are skipped whole)
    int sb = bb;
    if (slots) {
        sb = slots[bb];
        if (sb < 0 || sb >= n_slots) return;
    }
    // state slice in registers
    float S[R][4];
    const long sbase = ((long)sb * H + hh) * DK * DV;
    if (S0) {
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const float4 s = *reinterpret_cast<const float4*>(S0 + sbase + (long)(row0 + m) * DV + col0);
            S[m][0] = s.x; S[m][1] = s.y; S[m][2] = s.z; S[m][3] = s.w;
        }
    } else {
#pragma unroll
        for (int m = 0; m < R; ++m) S[m][0] = S[m][1] = S[m][2] = S[m][3] = 0.f;
    }

    auto fetch = [&](int t, float* qx, float* kx, float* ax, float* bx, float* vx, float* wx) {
        const long tok = ((long)bb * T + t) * H + hh;
        load_vec<R, BF16>(q, tok * DK + row0, qx);
        load_vec<R, BF16>(k, tok * DK + row0, kx);
        if constexpr (ASCALAR) {
            const float a = load_one<BF16>(alpha, tok);
#pragma unroll
            for (int m = 0; m < R; ++m) ax[m] = a;
        } else {
            load_vec<R, BF16>(alpha, tok * DK + row0, ax);
        }
        load_vec<4, BF16>(v, tok * DV + col0, vx);
        if constexpr (BSCALAR) {
            const float be = load_one<BF16>(b, tok);
#pragma unroll
            for (int m = 0; m < R; ++m) bx[m] = be;
#pragma unroll
            for (int c = 0; c < 4; ++c) wx[c] = be;
        } else {
            load_vec<R, BF16>(b, tok * DK + row0, bx);
            load_vec<4, BF16>(w, tok * DV + col0, wx);
        }
        if constexpr ((PRO & 2) != 0) {
#pragma unroll
            for (int m = 0; m < R; ++m) {
                ax[m] = sigmoid(ax[m]);
                bx[m] = sigmoid(bx[m]);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) wx[c] = sigmoid(wx[c]);
        }
    };

    // one token: the two reductions, delta, the readout and the state update
    auto token = [&](int t, const float* qa, const float* ka, const float* aa, const float* ba, const float* va,
                     const float* wa) {
        float r[4] = {0.f, 0.f, 0.f, 0.f}, po[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f, sq = 0.f, sk = 0.f;
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const float e = aa[m] * ba[m] * ka[m];
            const float aq = aa[m] * qa[m];
            qk = fmaf(qa[m], ka[m], qk);
            if constexpr ((PRO & 1) != 0) {
                sq = fmaf(qa[m], qa[m], sq);
                sk = fmaf(ka[m], ka[m], sk);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                r[c] = fmaf(e, S[m][c], r[c]);
                po[c] = fmaf(aq, S[m][c], po[c]);
            }
        }
        // sum over the 8 row groups (lane bits 3..5)
#pragma unroll
        for (int sh = 8; sh < kWave; sh <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                r[c] += __shfl_xor(r[c], sh);
                po[c] += __shfl_xor(po[c], sh);
            }
            qk += __shfl_xor(qk, sh);
            if constexpr ((PRO & 1) != 0) {
                sq += __shfl_xor(sq, sh);
                sk += __shfl_xor(sk, sh);
            }
        }
        float nk = 1.f;
        if constexpr ((PRO & 1) != 0) {
            nk = 1.f / fmaxf(sqrtf(sk), 1e-12f);
            const float nq = 1.f / fmaxf(sqrtf(sq), 1e-12f);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                r[c] *= nk;
                po[c] *= nq;
            }
            qk *= nq * nk;
        }
        float delta[4], oc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            delta[c] = fmaf(wa[c], va[c], -r[c]);
            oc[c] = fmaf(qk, delta[c], po[c]);
        }
#pragma unroll
        for (int m = 0; m < R; ++m) {
#pragma unroll
            for (int c = 0; c < 4; ++c) S[m][c] = fmaf(aa[m], S[m][c], (ka[m] * nk) * delta[c]);
        }
        if (rg == 0) {
            const long tok = ((long)bb * T + t) * H + hh;
            *reinterpret_cast<float4*>(o + tok * DV + col0) = make_float4(oc[0], oc[1], oc[2], oc[3]);
        }
    };

    if constexpr (ONE) {
        float qa[R], ka[R], aa[R], ba[R], va[4], wa[4];
        fetch(0, qa, ka, aa, ba, va, wa);
        token(0, qa, ka, aa, ba, va, wa);
    } else {
        // per-token inputs for this lane (current and next, for prefetch)
        float qa[R], ka[R], aa[R], ba[R], va[4], wa[4];
        float qn[R], kn[R], an[R], bn[R], vn[4], wn[4];
        if (T > 0) fetch(0, qa, ka, aa, ba, va, wa);
        for (int t = 0; t < T; ++t) {
            if (t + 1 < T) fetch(t + 1, qn, kn, an, bn, vn, wn);
            token(t, qa, ka, aa, ba, va, wa);
            if (t + 1 < T) {
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    qa[m] = qn[m]; ka[m] = kn[m]; aa[m] = an[m]; ba[m] = bn[m];
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) { va[c] = vn[c]; wa[c] = wn[c]; }
            }
        }
    }

    if (S_out) {
#pragma unroll
        for (int m = 0; m < R; ++m) {
            *reinterpret_cast<float4*>(S_out + sbase + (long)(row0 + m) * DV + col0) =
                make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
        }
    }
}

template <int DK, bool BF16, bool AS, bool BS, int PRO>
hipError_t launch_t(const RecurrentArgs& a, hipStream_t s) {
    const int items = a.B * a.H * (a.DV / 32);
    // A decode step (T = 1) whose states fit in the 256 MB Infinity Cache runs the one-token kernel
    // with two waves per workgroup: step after step the state largely stays in that cache, and
    // finer workgroups with more of them per SIMD stream it faster (B256 H16 d128, 256 MiB:
    // 87.0 us against 93.0 us for the general kernel with one wave per workgroup and 102.8 us with
    // four). Past about 400 MB of state the cache no longer holds it and the general kernel with
    // four waves per workgroup is faster, at its two waves per SIMD (B1024: 383 us against 399 us
    // for the one-token kernel held to the same occupancy and 410 us at its own three per SIMD;
    // 423 us with one wave per workgroup); so also the token-by-token prefill.
    const size_t state_bytes = (size_t)a.B * a.H * DK * a.DV * 4;
    const bool cached = a.T == 1 && state_bytes <= (size_t(320) << 20);
    const int waves_per_block = cached ? 2 : 4;
    const int blocks = (items + waves_per_block - 1) / waves_per_block;
    if (cached)
        hipLaunchKernelGGL((recurrent_kernel<DK, BF16, AS, BS, PRO, true>), dim3(blocks), dim3(64 * waves_per_block),
                           0, s, a.q, a.k, a.v, a.alpha, a.b, a.w, a.S0, a.o, a.S_out, a.B, a.T, a.H,
                           a.DV, a.slots, a.n_slots);
    else
        hipLaunchKernelGGL((recurrent_kernel<DK, BF16, AS, BS, PRO, false>), dim3(blocks), dim3(64 * waves_per_block),
                           0, s, a.q, a.k, a.v, a.alpha, a.b, a.w, a.S0, a.o, a.S_out, a.B, a.T, a.H,
                           a.DV, a.slots, a.n_slots);
    return hipGetLastError();
}

template <int DK, bool BF16, int PRO>
hipError_t launch_gates(const RecurrentArgs& a, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_t<DK, BF16, false, false, PRO>(a, s);
        case 1: return launch_t<DK, BF16, true, false, PRO>(a, s);
        case 2: return launch_t<DK, BF16, false, true, PRO>(a, s);
        default: return launch_t<DK, BF16, true, true, PRO>(a, s);
    }
}

template <int DK, bool BF16>
hipError_t launch_flags(const RecurrentArgs& a, hipStream_t s) {
    switch ((a.flags >> 2) & 3u) {  // prologue: L2 norm of q, k (1), gate pre-activations (2)
        case 0: return launch_gates<DK, BF16, 0>(a, s);
        case 1: return launch_gates<DK, BF16, 1>(a, s);
        case 2: return launch_gates<DK, BF16, 2>(a, s);
        default: return launch_gates<DK, BF16, 3>(a, s);
    }
}

template <int DK>
hipError_t launch_dtype(const RecurrentArgs& a, hipStream_t s) {
    return a.bf16 ? launch_flags<DK, true>(a, s) : launch_flags<DK, false>(a, s);
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s) {
    switch (a.DK) {
        case 32: return launch_dtype<32>(a, s);
        case 64: return launch_dtype<64>(a, s);
        case 128: return launch_dtype<128>(a, s);
        case 256: return launch_dtype<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn2
