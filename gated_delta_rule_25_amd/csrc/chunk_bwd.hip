// chunk_bwd.hip -- backward pass of the chunkwise (C = 64) Gated DeltaNet-2 prefill on gfx950.
//
// The gradients of L = sum_t <dO_t, o_t> + <dS_T, S_T> with respect to q, k, v, alpha, b, w and S0,
// for the recurrence S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T, o_t =
// S_t^T q_t [page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph
// "Техническая схема", state-update equation], through the chunkwise form the forward uses
// [same page, paragraph "Реализация": WY form, C = 64, decay absorbed into the rank-1 factors].
//
// Per chunk (64 rows r, s; key channels i; value channels j), with the chunk's start state S and
// the forward quantities of the operand block (Q_hat = q e^G, E_hat = (b*k) e^G, K_bar = k
// e^(G_C - G), gamma = e^(G_C), P, T = (I + A)^-1, G the in-chunk cumulative log-decay):
//     D' = U - E_hat S,  Delta = T D',  O = Q_hat S + P Delta,  S_end = Diag(gamma) S + K_bar^T Delta.
// Reverse mode, with G' = dL/dS_end:
//     dDelta = P^T dO + K_bar G',   dD' = T^T dDelta,   dU = dD' (dv = w*dD', dw = v*dD'),
//     dL/dS  = Q_hat^T dO + Diag(gamma) G' - E_hat^T dD'                  (carried to chunk n-1),
//     dQ_hat = dO S^T,  dE_hat = -dD' S^T,  dK_bar = Delta G'^T,  dgamma_i = sum_j S_ij G'_ij,
//     dP = dO Delta^T (lower),  dA = -T^T (dDelta D'^T) T^T (strictly lower),
// then through the factors: with F_rsi = prod_{m=s+1..r} alpha_mi (= e^(G_ri - G_si), never above 1)
//     XA_ri = sum_{s<r} dA_rs k_si F_rsi,   XP_ri = sum_{s<=r} dP_rs k_si F_rsi,
//     Y_si  = sum_{r>s} dA_rs (b*k)_ri F_rsi + sum_{r>=s} dP_rs q_ri F_rsi,
//     dq = dQ_hat e^G + XP,  d(b*k) = dE_hat e^G + XA,  dk = dK_bar e^(G_C-G) + Y + b d(b*k),
//     db = k d(b*k),  dG_ri = dQ_hat Q_hat + dE_hat E_hat - dK_bar K_bar + (b*k) XA + q XP - k Y
//     (plus, on the last row, sum_r dK_bar K_bar + dgamma gamma), dlog(alpha)_s = sum_{r>=s} dG_r.
//
// Kernels, in order (all on the caller's stream):
//   1. prep + state-only chain (chunk_split.hip): the operand blocks, the start state of every
//      chunk, and the rows of D' and Delta.
//   2. bwd_chain_kernel: dL/dS backwards over the chunks, one workgroup per (b, h, 64 value
//      columns), the gradient state in MFMA accumulators; writes G' of every chunk, dDelta, dD',
//      dv, dw and dS0.
//   3. bwd_contract_kernel: per (b, h, chunk), the products contracted over the value channels
//      (dQ_hat, dE_hat, dK_bar, dgamma, dP) and dA, in fp32.
//   4. bwd_key_kernel: per (b, h, chunk), the decay-weighted sums XA, XP, Y by running products
//      of alpha, the elementwise terms and the reverse cumulative sum; writes dq, dk, db, dalpha.
#include "chunk_blob.h"
#include "kernels.h"

namespace gdn2 {

namespace {

using namespace chunk;

__device__ __forceinline__ float bload_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ float bload_bf16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0) << 16);
}
__device__ __forceinline__ void bstore_f32(__amdgpu_buffer_rsrc_t r, unsigned off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)off, 0, 0);
}

// Element (r, c) of T or P in an fp16 operand block: blocks the block does not store (columns
// 32..63 of rows 0..31) are zero.
template <typename BL>
__device__ __forceinline__ float tp_get(const _Float16* X, int r, int c) {
    return (r < 32 && c >= 32) ? 0.f : (float)X[BL::tp(r, c)];
}

// ------------------------------------------------------------------------------------------
// 2. reverse chain
struct ChainBwdIO {
    const void* v;
    const void* w;
    const float* dO;    // [B, T, H, DV]
    const float* dS_T;  // [B, H, DK, DV] or null
    const char* blobs;  // [b*h][nch] operand blocks
    float* G_save;      // [b*h][nch][DK][DV]: dL/dS at the end of each chunk
    float* dDl;         // [B, T, H, DV]: dL/dDelta
    float* dDp;         // [B, T, H, DV]: dL/dD'
    float* dv;
    float* dw;
    float* dS0;  // [B, H, DK, DV] or null
    int B, T, H, DV, nch;
};

template <int DK>
__global__ void __launch_bounds__(256, 1) bwd_chain_kernel(const ChainBwdIO io) {
    using PR = Prec<true>;
    using E = _Float16;
    using Frag = PR::Frag;
    using BL = Blob<DK, true>;
    constexpr int NKS = DK / 32, NMK = DK / 16;
    constexpr int DVT = DK < 64 ? DK : 64;
    constexpr int NW = DVT / 16;  // waves, 16 value columns each

    __shared__ __attribute__((aligned(16))) char smem[BL::bytes];
    const E* En = reinterpret_cast<const E*>(smem + BL::oEn);
    const E* KbT = reinterpret_cast<const E*>(smem + BL::oKbT);
    const E* Tm = reinterpret_cast<const E*>(smem + BL::oTm);
    const E* Pm = reinterpret_cast<const E*>(smem + BL::oP);
    const E* Qh = reinterpret_cast<const E*>(smem + BL::oQh);
    const float* gC = reinterpret_cast<const float*>(smem + BL::oGC);

    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int H = io.H, T = io.T, DV = io.DV, nch = io.nch;
    const int vt = DV / DVT;
    const int bh = blockIdx.x / vt, tile = blockIdx.x % vt;
    const int hh = bh % H, bb = bh / H;
    const int col = tile * DVT + 16 * wv + l16;

    const long seq = (long)bb * T * H;
    const unsigned seq_f32 = (unsigned)T * H * DV * 4u;
    const auto rs_dO = make_rsrc(io.dO + seq * DV, seq_f32);
    const auto rs_dDl = make_rsrc(io.dDl + seq * DV, seq_f32);
    const auto rs_dDp = make_rsrc(io.dDp + seq * DV, seq_f32);
    const auto rs_dv = make_rsrc(io.dv + seq * DV, seq_f32);
    const auto rs_dw = make_rsrc(io.dw + seq * DV, seq_f32);
    const auto rs_v = make_rsrc(static_cast<const uint16_t*>(io.v) + seq * DV, (unsigned)T * H * DV * 2u);
    const auto rs_w = make_rsrc(static_cast<const uint16_t*>(io.w) + seq * DV, (unsigned)T * H * DV * 2u);
    // element index of (token row 0 of the sequence, head hh, column col)
    auto elem = [&](int row) -> unsigned { return ((unsigned)row * H + hh) * DV + col; };

    // G: dL/dS for this wave's 16 columns; [mk][j] is row 16 mk + 4 g + j, column col
    f4 G[NMK];
#pragma unroll
    for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            G[mk][j] = io.dS_T ? io.dS_T[((size_t)bh * DK + 16 * mk + 4 * g + j) * DV + col] : 0.f;

    auto stack = [](const f4& lo, const f4& hi) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t[i] = lo[i];
            t[i + 4] = hi[i];
        }
        return PR::make(t);
    };

    for (int n = nch - 1; n >= 0; --n) {
        const int t0 = n * CH;
        lds_barrier();  // every read of the previous block is done
        dma_flat(io.blobs + ((size_t)bh * nch + n) * BL::bytes, smem, BL::bytes, wv, NW, lane);
        wait_dma();
        lds_barrier();

        // G' of this chunk, for the contraction kernel
        float* gs = io.G_save + ((size_t)bh * nch + n) * DK * DV;
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
            for (int j = 0; j < 4; ++j) gs[(size_t)(16 * mk + 4 * g + j) * DV + col] = G[mk][j];

        // dO of the chunk's rows as B operands (k = token row, n = column); rows past T are zero
        Frag dOf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = bload_f32(rs_dO, elem(t0 + 32 * s2 + kap(g, i)) * 4u);
            dOf[s2] = PR::make(x);
        }
        Frag Gf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) Gf[s] = stack(G[2 * s], G[2 * s + 1]);

        // dDelta = P^T dO + K_bar G'   (P^T[r][s] = P[s][r] is zero for s < r)
        f4 dL[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            dL[mt] = f4{0.f, 0.f, 0.f, 0.f};
            const int m = 16 * mt + l16;
#pragma unroll
            for (int s2 = mt / 2; s2 < 2; ++s2) {
                float a[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = tp_get<BL>(Pm, 32 * s2 + kap(g, i), m);
                PR::mma(dL[mt], PR::make(a), dOf[s2]);
            }
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                float a[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = (float)KbT[BL::kbt(32 * s + kap(g, i), m)];
                PR::mma(dL[mt], PR::make(a), Gf[s]);
            }
        }
        // dD' = T^T dDelta
        const Frag dLf[2] = {stack(dL[0], dL[1]), stack(dL[2], dL[3])};
        f4 dP[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            dP[mt] = f4{0.f, 0.f, 0.f, 0.f};
            const int m = 16 * mt + l16;
#pragma unroll
            for (int s2 = mt / 2; s2 < 2; ++s2) {
                float a[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = tp_get<BL>(Tm, 32 * s2 + kap(g, i), m);
                PR::mma(dP[mt], PR::make(a), dLf[s2]);
            }
        }
        // rows of dDelta and dD'; dv = w dD', dw = v dD' (rows past T are dropped)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned e = elem(t0 + 16 * mt + 4 * g + j);
                bstore_f32(rs_dDl, e * 4u, dL[mt][j]);
                bstore_f32(rs_dDp, e * 4u, dP[mt][j]);
                const float vv = bload_bf16(rs_v, e * 2u), ww = bload_bf16(rs_w, e * 2u);
                bstore_f32(rs_dv, e * 4u, ww * dP[mt][j]);
                bstore_f32(rs_dw, e * 4u, vv * dP[mt][j]);
            }
        // dL/dS at the chunk start = Q_hat^T dO + Diag(gamma) G' - E_hat^T dD'  (En = -E_hat)
        const Frag dPf[2] = {stack(dP[0], dP[1]), stack(dP[2], dP[3])};
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk) {
            const int m = 16 * mk + l16;
#pragma unroll
            for (int j = 0; j < 4; ++j) G[mk][j] *= gC[16 * mk + 4 * g + j];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float aq[8], ae[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 32 * s2 + kap(g, i);
                    aq[i] = (float)Qh[BL::en(r, m)];
                    ae[i] = (float)En[BL::en(r, m)];
                }
                PR::mma(G[mk], PR::make(aq), dOf[s2]);
                PR::mma(G[mk], PR::make(ae), dPf[s2]);
            }
        }
    }
    if (io.dS0) {
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
            for (int j = 0; j < 4; ++j) io.dS0[((size_t)bh * DK + 16 * mk + 4 * g + j) * DV + col] = G[mk][j];
    }
}

// ------------------------------------------------------------------------------------------
// 3. contractions over the value channels, per (b, h, chunk)
struct ContractIO {
    const float* dO;   // [B, T, H, DV]
    const float* Dp;   // D'
    const float* Dl;   // Delta
    const float* dDl;  // dDelta
    const float* dDp;  // dD'
    const float* S_save;
    const float* G_save;
    const char* blobs;
    float* dQh;  // [b*h][nch][64][DK]
    float* dEh;
    float* dKb;
    float* dPm;  // [b*h][nch][64][64]
    float* dAm;
    float* dgam;  // [b*h][nch][DK]
    int B, T, H, DV, nch;
};

template <int DK>
__global__ void __launch_bounds__(256, 2) bwd_contract_kernel(const ContractIO io) {
    using BL = Blob<DK, true>;
    constexpr int JS = 32, JP = JS + 1;  // value columns per slice, padded row
    constexpr int CPT = DK / 16;         // key channels per thread
    constexpr int SM = (2 * DK + 5 * CH) * JP;
    static_assert(SM >= 3 * CH * (CH + 1), "the UT adjoint reuses the slice buffers");
    __shared__ float lds[SM];
    float* Ss = lds;              // [DK][JP]
    float* Gs = Ss + DK * JP;     // [DK][JP]
    float* dOs = Gs + DK * JP;    // [64][JP]
    float* dDps = dOs + CH * JP;  // [64][JP]
    float* Dls = dDps + CH * JP;
    float* dDls = Dls + CH * JP;
    float* Dps = dDls + CH * JP;

    const int tid = threadIdx.x;
    const int H = io.H, T = io.T, DV = io.DV, nch = io.nch;
    const int bh = blockIdx.x / nch, n = blockIdx.x % nch;
    const int hh = bh % H, bb = bh / H;
    const int t0 = n * CH;
    const int rb = tid / 16, cb = tid % 16;  // rows 4 rb .. 4 rb + 3
    const float* S = io.S_save + ((size_t)bh * nch + n) * DK * DV;
    const float* Gp = io.G_save + ((size_t)bh * nch + n) * DK * DV;

    float aQ[4][CPT] = {}, aE[4][CPT] = {}, aK[4][CPT] = {}, aP[4][4] = {}, aT[4][4] = {};
    float ag = 0.f;
    for (int js = 0; js < DV; js += JS) {
        __syncthreads();
        for (int x = tid; x < DK * JS; x += 256) {
            const int i = x / JS, j = x % JS;
            Ss[i * JP + j] = S[(size_t)i * DV + js + j];
            Gs[i * JP + j] = Gp[(size_t)i * DV + js + j];
        }
        for (int x = tid; x < CH * JS; x += 256) {
            const int r = x / JS, j = x % JS;
            const int t = t0 + r;
            const bool ok = t < T;
            const size_t e = (((size_t)bb * T + (ok ? t : 0)) * H + hh) * DV + js + j;
            dOs[r * JP + j] = ok ? io.dO[e] : 0.f;
            dDps[r * JP + j] = ok ? io.dDp[e] : 0.f;
            Dls[r * JP + j] = ok ? io.Dl[e] : 0.f;
            dDls[r * JP + j] = ok ? io.dDl[e] : 0.f;
            Dps[r * JP + j] = ok ? io.Dp[e] : 0.f;
        }
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < JS; ++j) {
            float o4[4], e4[4], l4[4], d4[4], lc[4], pc[4], s8[CPT], g8[CPT];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 4 * rb + q;
                o4[q] = dOs[r * JP + j];
                e4[q] = dDps[r * JP + j];
                l4[q] = Dls[r * JP + j];
                d4[q] = dDls[r * JP + j];
                lc[q] = Dls[(4 * cb + q) * JP + j];
                pc[q] = Dps[(4 * cb + q) * JP + j];
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                s8[c] = Ss[(CPT * cb + c) * JP + j];
                g8[c] = Gs[(CPT * cb + c) * JP + j];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    aQ[q][c] = fmaf(o4[q], s8[c], aQ[q][c]);
                    aE[q][c] = fmaf(-e4[q], s8[c], aE[q][c]);
                    aK[q][c] = fmaf(l4[q], g8[c], aK[q][c]);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    aP[q][c] = fmaf(o4[q], lc[c], aP[q][c]);
                    aT[q][c] = fmaf(d4[q], pc[c], aT[q][c]);
                }
            }
        }
        if (tid < DK) {
            for (int j = 0; j < JS; ++j) ag = fmaf(Ss[tid * JP + j], Gs[tid * JP + j], ag);
        }
    }
    const size_t cbase = ((size_t)bh * nch + n);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 4 * rb + q;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const size_t e = (cbase * CH + r) * DK + CPT * cb + c;
            io.dQh[e] = aQ[q][c];
            io.dEh[e] = aE[q][c];
            io.dKb[e] = aK[q][c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int cc = 4 * cb + c;
            io.dPm[(cbase * CH + r) * CH + cc] = cc <= r ? aP[q][c] : 0.f;
        }
    }
    if (tid < DK) io.dgam[cbase * DK + tid] = ag;

    // dA = -T^T dT T^T (strictly lower), dT = dDelta D'^T on the lower triangle
    __syncthreads();
    constexpr int TP = CH + 1;
    float* Tf = lds;            // [64][TP] T
    float* Tg = Tf + CH * TP;   // [64][TP] dT
    float* Xm = Tg + CH * TP;   // [64][TP] T^T dT
    const _Float16* Tb = reinterpret_cast<const _Float16*>(io.blobs + cbase * BL::bytes + BL::oTm);
    for (int x = tid; x < CH * CH; x += 256) {
        const int r = x / CH, c = x % CH;
        Tf[r * TP + c] = tp_get<BL>(Tb, r, c);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r = 4 * rb + q, cc = 4 * cb + c;
            Tg[r * TP + cc] = cc <= r ? aT[q][c] : 0.f;
        }
    __syncthreads();
    // X = T^T dT: X[r][c] = sum_m T[m][r] dT[m][c]
    float xacc[4][4] = {};
    for (int m = 0; m < CH; ++m) {
        float tr[4], tc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            tr[q] = Tf[m * TP + 4 * rb + q];
            tc[q] = Tg[m * TP + 4 * cb + q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) xacc[q][c] = fmaf(tr[q], tc[c], xacc[q][c]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) Xm[(4 * rb + q) * TP + 4 * cb + c] = xacc[q][c];
    __syncthreads();
    // dA[r][c] = -sum_m X[r][m] T[c][m], kept for c < r
    float dacc[4][4] = {};
    for (int m = 0; m < CH; ++m) {
        float xr[4], tc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xr[q] = Xm[(4 * rb + q) * TP + m];
            tc[q] = Tf[(4 * cb + q) * TP + m];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) dacc[q][c] = fmaf(xr[q], tc[c], dacc[q][c]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r = 4 * rb + q, cc = 4 * cb + c;
            io.dAm[(cbase * CH + r) * CH + cc] = cc < r ? -dacc[q][c] : 0.f;
        }
}

// ------------------------------------------------------------------------------------------
// 4. key side, per (b, h, chunk)
struct KeyIO {
    const void *q, *k, *alpha, *b;  // bf16 [B, T, H, DK]
    const float *dQh, *dEh, *dKb, *dPm, *dAm, *dgam;
    float *dq, *dk, *dalpha, *db;  // [B, T, H, DK]
    int B, T, H, nch;
};

template <int DK>
__global__ void __launch_bounds__(256, 1) bwd_key_kernel(const KeyIO io) {
    constexpr int AP = CH + 1;
    constexpr int R = 256 / DK;  // row phases: thread (i, h) owns rows h, h + R, ...
    __shared__ uint16_t qs[CH * DK], ks[CH * DK], bs[CH * DK], as[CH * DK];
    __shared__ float dA[CH * AP], dPs[CH * AP];
    __shared__ float Gm[CH * DK];  // cumulative log2 decay, then dL/dG
    __shared__ float red[256];

    const int tid = threadIdx.x;
    const int H = io.H, T = io.T, nch = io.nch;
    const int bh = blockIdx.x / nch, n = blockIdx.x % nch;
    const int hh = bh % H, bb = bh / H;
    const int t0 = n * CH;
    const size_t cbase = (size_t)bh * nch + n;
    const uint16_t* q = static_cast<const uint16_t*>(io.q);
    const uint16_t* k = static_cast<const uint16_t*>(io.k);
    const uint16_t* al = static_cast<const uint16_t*>(io.alpha);
    const uint16_t* b = static_cast<const uint16_t*>(io.b);
    for (int x = tid; x < CH * DK; x += 256) {
        const int r = x / DK, i = x % DK;
        const int t = t0 + r;
        const bool ok = t < T;
        const size_t e = (((size_t)bb * T + (ok ? t : 0)) * H + hh) * DK + i;
        qs[x] = ok ? q[e] : 0;
        ks[x] = ok ? k[e] : 0;
        bs[x] = ok ? b[e] : 0;
        as[x] = ok ? al[e] : (uint16_t)0x3F80;  // 1.0: rows past the end do not decay
    }
    for (int x = tid; x < CH * CH; x += 256) {
        const int r = x / CH, c = x % CH;
        dA[r * AP + c] = io.dAm[cbase * CH * CH + x];
        dPs[r * AP + c] = io.dPm[cbase * CH * CH + x];
    }
    __syncthreads();
    auto f = [](uint16_t x) { return __uint_as_float((uint32_t)x << 16); };
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < CH; ++r) {
            acc += __builtin_amdgcn_logf(f(as[r * DK + tid]));
            Gm[r * DK + tid] = acc;
        }
    }
    __syncthreads();

    const int i = tid % DK, h = tid / DK;
    const float G63 = Gm[(CH - 1) * DK + i];
    constexpr int NR = CH / R;
    float dG[NR];
    float kb_sum = 0.f;
    for (int m = 0; m < NR; ++m) {
        const int r = h + R * m;
        const float kr = f(ks[r * DK + i]), qr = f(qs[r * DK + i]), br = f(bs[r * DK + i]);
        // XA, XP: sums over s <= r, F = prod_{m = s+1..r} alpha_m
        float F = 1.f, XA = 0.f, XP = dPs[r * AP + r] * kr;
        for (int s = r - 1; s >= 0; --s) {
            F *= f(as[(s + 1) * DK + i]);
            const float kf = f(ks[s * DK + i]) * F;
            XA = fmaf(dA[r * AP + s], kf, XA);
            XP = fmaf(dPs[r * AP + s], kf, XP);
        }
        // Y: sums over r2 >= r, F = prod_{m = r+1..r2} alpha_m
        float Y = dPs[r * AP + r] * qr;
        F = 1.f;
        for (int r2 = r + 1; r2 < CH; ++r2) {
            F *= f(as[r2 * DK + i]);
            const float k2 = f(ks[r2 * DK + i]);
            Y = fmaf(fmaf(dA[r2 * AP + r], f(bs[r2 * DK + i]) * k2, dPs[r2 * AP + r] * f(qs[r2 * DK + i])), F, Y);
        }
        const float G2 = Gm[r * DK + i];
        const float eG = __builtin_amdgcn_exp2f(G2), eK = __builtin_amdgcn_exp2f(G63 - G2);
        const size_t ce = (cbase * CH + r) * DK + i;
        const float gQ = io.dQh[ce], gE = io.dEh[ce], gK = io.dKb[ce];
        const float Et = br * kr;
        const float dEt = fmaf(gE, eG, XA);
        const float dqv = fmaf(gQ, eG, XP);
        const float dkv = fmaf(gK, eK, Y) + br * dEt;
        const float dbv = kr * dEt;
        dG[m] = gQ * qr * eG + gE * Et * eG - gK * kr * eK + Et * XA + qr * XP - kr * Y;
        kb_sum = fmaf(gK, kr * eK, kb_sum);
        const int t = t0 + r;
        if (t < T) {
            const size_t e = (((size_t)bb * T + t) * H + hh) * DK + i;
            io.dq[e] = dqv;
            io.dk[e] = dkv;
            io.db[e] = dbv;
        }
    }
    red[tid] = kb_sum;
    __syncthreads();  // every read of Gm is done
#pragma unroll
    for (int m = 0; m < NR; ++m) Gm[(h + R * m) * DK + i] = dG[m];
    __syncthreads();
    if (tid < DK) {
        float extra = io.dgam[cbase * DK + i] * __builtin_amdgcn_exp2f(G63);
        for (int p = 0; p < R; ++p) extra += red[p * DK + i];
        // dlog(alpha)_s = sum_{r >= s} dG_r (the last row also carries the gamma and K_bar terms)
        float acc = extra;
        for (int r = CH - 1; r >= 0; --r) {
            acc += Gm[r * DK + i];
            const int t = t0 + r;
            if (t < T) {
                const size_t e = (((size_t)bb * T + t) * H + hh) * DK + i;
                io.dalpha[e] = acc / f(as[r * DK + i]);
            }
        }
    }
}

__global__ void __launch_bounds__(256) copy_or_zero(float* dst, const float* src, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

struct BwdLayout {
    size_t blobs, S_save, G_save, Dp, Dl, dDl, dDp, dQh, dEh, dKb, dPm, dAm, dgam, total;
};

BwdLayout bwd_layout(int B, int T, int H, int DK, int DV) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t BH = (size_t)B * H, nch = ((size_t)T + CH - 1) / CH;
    BwdLayout L{};
    size_t o = 0;
    L.blobs = o;
    o += up(nch * split_chunk_bytes(B, H, DK, true));
    const size_t st = up(BH * nch * DK * DV * 4);
    L.S_save = o;
    o += st;
    L.G_save = o;
    o += st;
    const size_t rows = up((size_t)B * T * H * DV * 4);
    L.Dp = o;
    o += rows;
    L.Dl = o;
    o += rows;
    L.dDl = o;
    o += rows;
    L.dDp = o;
    o += rows;
    const size_t kr = up(BH * nch * CH * DK * 4);
    L.dQh = o;
    o += kr;
    L.dEh = o;
    o += kr;
    L.dKb = o;
    o += kr;
    const size_t pm = up(BH * nch * CH * CH * 4);
    L.dPm = o;
    o += pm;
    L.dAm = o;
    o += pm;
    L.dgam = o;
    o += up(BH * nch * DK * 4);
    L.total = o;
    return L;
}

template <int DK>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
    const BwdLayout L = bwd_layout(a.B, a.T, a.H, DK, a.DV);
    char* ws = static_cast<char*>(a.workspace);
    const int BH = a.B * a.H, nch = (a.T + CH - 1) / CH;
    char* blobs = ws + L.blobs;
    float* S_save = reinterpret_cast<float*>(ws + L.S_save);
    float* G_save = reinterpret_cast<float*>(ws + L.G_save);
    float* Dp = reinterpret_cast<float*>(ws + L.Dp);
    float* Dl = reinterpret_cast<float*>(ws + L.Dl);
    float* dDl = reinterpret_cast<float*>(ws + L.dDl);
    float* dDp = reinterpret_cast<float*>(ws + L.dDp);
    float* dQh = reinterpret_cast<float*>(ws + L.dQh);
    float* dEh = reinterpret_cast<float*>(ws + L.dEh);
    float* dKb = reinterpret_cast<float*>(ws + L.dKb);
    float* dPm = reinterpret_cast<float*>(ws + L.dPm);
    float* dAm = reinterpret_cast<float*>(ws + L.dAm);
    float* dgam = reinterpret_cast<float*>(ws + L.dgam);

    const ChunkArgs fa{a.q, a.k, a.v, a.alpha, a.b, a.w, a.S0, nullptr, nullptr, a.B, a.T, a.H, DK, a.DV,
                       true, 0u, nullptr, 0};
    hipError_t e = launch_split_states(fa, blobs, S_save, Dp, Dl, st);
    if (e != hipSuccess) return e;

    constexpr int DVT = DK < 64 ? DK : 64;
    const ChainBwdIO cio{a.v, a.w, a.dO, a.dS_T, blobs, G_save, dDl, dDp, a.dv, a.dw, a.dS0,
                         a.B, a.T, a.H, a.DV, nch};
    hipLaunchKernelGGL((bwd_chain_kernel<DK>), dim3(BH * (a.DV / DVT)), dim3(64 * (DVT / 16)), 0, st, cio);
    const ContractIO xio{a.dO, Dp, Dl, dDl, dDp, S_save, G_save, blobs, dQh, dEh, dKb, dPm, dAm, dgam,
                         a.B, a.T, a.H, a.DV, nch};
    hipLaunchKernelGGL((bwd_contract_kernel<DK>), dim3(BH * nch), dim3(256), 0, st, xio);
    const KeyIO kio{a.q, a.k, a.alpha, a.b, dQh, dEh, dKb, dPm, dAm, dgam, a.dq, a.dk, a.dalpha, a.db,
                    a.B, a.T, a.H, nch};
    hipLaunchKernelGGL((bwd_key_kernel<DK>), dim3(BH * nch), dim3(256), 0, st, kio);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int T, int H, int DK, int DV, bool bf16, uint32_t flags) {
    if (!bf16 || flags != 0u || DK != DV) return false;
    if (DK != 32 && DK != 64 && DK != 128) return false;
    // one sequence's rows, the last chunk's rows past T included, addressed with 32-bit offsets
    return ((long long)T + CH) * H * DV * 4 < (1ll << 32);
}

size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV) { return bwd_layout(B, T, H, DK, DV).total; }

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
    if (!bwd_supported(a.T, a.H, a.DK, a.DV, a.bf16, a.flags)) return hipErrorNotSupported;
    if (a.T == 0) {  // no tokens: dS0 = dS_T (or zeros), nothing else to write
        if (!a.dS0) return hipSuccess;
        const long n = (long)a.B * a.H * a.DK * a.DV;
        hipLaunchKernelGGL(copy_or_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.dS0, a.dS_T, n);
        return hipGetLastError();
    }
    if (!a.workspace || a.workspace_bytes < bwd_workspace_bytes(a.B, a.T, a.H, a.DK, a.DV)) return hipErrorInvalidValue;
    switch (a.DK) {
        case 32: return launch_bwd_t<32>(a, s);
        case 64: return launch_bwd_t<64>(a, s);
        default: return launch_bwd_t<128>(a, s);
    }
}

}  // namespace gdn2
