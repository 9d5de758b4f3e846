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
// then through the factors: with F_rsi = prod_{m=s+1..r} alpha_mi (= e^(G_ri - G_si), at most 1)
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
//      (dQ_hat, dE_hat, dK_bar, dP, dT) on the matrix cores, dgamma, and dA in fp32.
//   4. bwd_key_kernel: per (b, h, chunk, 32 key channels), the decay-weighted sums XA, XP, Y
//      through block references (no factor above 1), the elementwise terms and the reverse
//      cumulative sum; writes dq, dk, db, dalpha.
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

// All five products contract over the value channels j with both operands row-major in j, the
// fragment layout of the matrix cores: fp16 operands (as in the chains), fp32 accumulation. The
// value channels are staged in slices of 64 columns; wave w owns output rows 16 w .. 16 w + 15.
template <int DK>
__global__ void __launch_bounds__(256, 2) bwd_contract_kernel(const ContractIO io) {
    using PR = Prec<true>;
    using E = _Float16;
    using Frag = PR::Frag;
    using BL = Blob<DK, true>;
    constexpr int JS = DK < 64 ? DK : 64;  // value columns per slice (d_v == d_k)
    constexpr int JP = JS + 4;    // row stride (halves): 2 dwords past a multiple of 32 banks
    constexpr int NMK = DK / 16;  // 16-channel tiles of the key axis
    constexpr int SMB = (2 * DK + 5 * CH) * JP * 2;  // bytes of one slice
    constexpr int TP = CH + 1;
    constexpr int UTB = 3 * CH * TP * 4;  // the UT adjoint reuses the slice buffers
    __shared__ __attribute__((aligned(16))) char lds[SMB > UTB ? SMB : UTB];
    E* Ss = reinterpret_cast<E*>(lds);  // [DK][JP]
    E* Gs = Ss + DK * JP;               // [DK][JP]
    E* dOs = Gs + DK * JP;              // [64][JP]: dO, dD', Delta, dDelta, D'
    E* dDps = dOs + CH * JP;
    E* Dls = dDps + CH * JP;
    E* dDls = Dls + CH * JP;
    E* Dps = dDls + CH * JP;

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int H = io.H, T = io.T, DV = io.DV, nch = io.nch;
    const int bh = blockIdx.x / nch, n = blockIdx.x % nch;
    const int hh = bh % H, bb = bh / H;
    const int t0 = n * CH;
    const size_t cbase = (size_t)bh * nch + n;
    const float* S = io.S_save + cbase * DK * DV;
    const float* Gp = io.G_save + cbase * DK * DV;

    f4 aQ[NMK], aE[NMK], aK[NMK], aP[4], aT[4];
#pragma unroll
    for (int c = 0; c < NMK; ++c) aQ[c] = aE[c] = aK[c] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) aP[c] = aT[c] = f4{0.f, 0.f, 0.f, 0.f};

    for (int js = 0; js < DV; js += JS) {
        __syncthreads();
        for (int x = tid; x < DK * JS / 4; x += 256) {
            const int i = x / (JS / 4), j = 4 * (x % (JS / 4));
            const float4 a = *reinterpret_cast<const float4*>(S + (size_t)i * DV + js + j);
            const float4 b = *reinterpret_cast<const float4*>(Gp + (size_t)i * DV + js + j);
            *reinterpret_cast<h4*>(Ss + i * JP + j) = h4{(E)a.x, (E)a.y, (E)a.z, (E)a.w};
            *reinterpret_cast<h4*>(Gs + i * JP + j) = h4{(E)b.x, (E)b.y, (E)b.z, (E)b.w};
        }
        for (int x = tid; x < CH * JS / 4; x += 256) {
            const int r = x / (JS / 4), j = 4 * (x % (JS / 4));
            const int t = t0 + r;
            const bool ok = t < T;
            const size_t e = (((size_t)bb * T + (ok ? t : 0)) * H + hh) * DV + js + j;
            const float* srcs[5] = {io.dO, io.dDp, io.Dl, io.dDl, io.Dp};
            E* dsts[5] = {dOs, dDps, Dls, dDls, Dps};
#pragma unroll
            for (int m = 0; m < 5; ++m) {
                float4 a = *reinterpret_cast<const float4*>(srcs[m] + e);
                if (!ok) a = make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<h4*>(dsts[m] + r * JP + j) = h4{(E)a.x, (E)a.y, (E)a.z, (E)a.w};
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < JS / 32; ++ks) {
            const int c0 = 32 * ks + 4 * g;
            auto frag = [&](const E* M, int row) { return PR::lds_pair(M + row * JP + c0, M + row * JP + c0 + 16); };
            const int r = 16 * wv + l16;
            const Frag fO = frag(dOs, r), fDp = frag(dDps, r), fL = frag(Dls, r), fdL = frag(dDls, r);
#pragma unroll
            for (int c = 0; c < NMK; ++c) {
                const Frag fS = frag(Ss, 16 * c + l16), fG = frag(Gs, 16 * c + l16);
                PR::mma(aQ[c], fO, fS);
                PR::mma(aE[c], fDp, fS);
                PR::mma(aK[c], fL, fG);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c <= wv) {
                    PR::mma(aP[c], fO, frag(Dls, 16 * c + l16));
                    PR::mma(aT[c], fdL, frag(Dps, 16 * c + l16));
                }
            }
        }
    }
    // accumulator [c][j]: row 16 wv + 4 g + j, column 16 c + l16
#pragma unroll
    for (int c = 0; c < NMK; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t e = (cbase * CH + 16 * wv + 4 * g + j) * DK + 16 * c + l16;
            io.dQh[e] = aQ[c][j];
            io.dEh[e] = -aE[c][j];
            io.dKb[e] = aK[c][j];
        }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wv + 4 * g + j, cc = 16 * c + l16;
            io.dPm[(cbase * CH + r) * CH + cc] = (c <= wv && cc <= r) ? aP[c][j] : 0.f;
        }
    // dgamma_i = sum_j S_ij G'_ij in fp32
    if (tid < DK) {
        float ag = 0.f;
        for (int j = 0; j < DV; j += 4) {
            const float4 a = *reinterpret_cast<const float4*>(S + (size_t)tid * DV + j);
            const float4 b = *reinterpret_cast<const float4*>(Gp + (size_t)tid * DV + j);
            ag += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
        }
        io.dgam[cbase * DK + tid] = ag;
    }

    // dA = -T^T dT T^T (strictly lower), dT = dDelta D'^T on the lower triangle
    __syncthreads();
    float* Tf = reinterpret_cast<float*>(lds);  // [64][TP] T
    float* Tg = Tf + CH * TP;                    // [64][TP] dT
    float* Xm = Tg + CH * TP;                    // [64][TP] T^T dT
    const _Float16* Tb = reinterpret_cast<const _Float16*>(io.blobs + cbase * BL::bytes + BL::oTm);
    for (int x = tid; x < CH * CH; x += 256) {
        const int r = x / CH, c = x % CH;
        Tf[r * TP + c] = tp_get<BL>(Tb, r, c);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wv + 4 * g + j, cc = 16 * c + l16;
            Tg[r * TP + cc] = (c <= wv && cc <= r) ? aT[c][j] : 0.f;
        }
    __syncthreads();
    const int rb = tid / 16, cb = tid % 16;  // 4 x 4 tile of rows 4 rb.., columns 4 cb..
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

// One workgroup per (b, h, chunk, 32 key channels): the decay-weighted sums are independent per
// channel. With G the cumulative log2 decay and 16-row blocks, a factor 2^(G_r - G_s) between
// blocks J < I splits at a row between them into two factors no larger than 1:
//   XA, XP (sum over s in J):  2^(G_r - G_e(J)) * [k_s 2^(G_e(J) - G_s)],   e(J) = last row of J,
//   Y      (sum over r in I):  [x_r 2^(G_r - G_b(I))] * 2^(G_b(I) - G_s),   b(I) = first row of I,
// so each block pair's sum is a 16x16 by 16x32 matrix product over pre-scaled rows (fp32 on the
// matrix cores) followed by one scale per output; inside a block the factor is taken directly
// (one exp2 per term, on the vector units).
template <int DK>
__global__ void __launch_bounds__(256, 2) bwd_key_kernel(const KeyIO io) {
    constexpr int CW = 32;       // key channels per workgroup
    constexpr int NG = DK / CW;  // channel groups
    static_assert(DK % CW == 0, "channel groups");
    __shared__ float dA[CH * CH], dPs[CH * CH];
    __shared__ float G2[CH * CW];                   // cumulative log2 decay
    __shared__ float Kp[CH * CW], Ep[CH * CW], Qp[CH * CW];  // pre-scaled rows (Kp then dL/dG)
    __shared__ uint16_t qs[CH * CW], ks[CH * CW], bs[CH * CW];
    __shared__ float red[8 * CW];

    const int tid = threadIdx.x;
    const int H = io.H, T = io.T, nch = io.nch;
    const int cg = blockIdx.x % NG, item = blockIdx.x / NG;
    const int bh = item / nch, n = item % nch;
    const int hh = bh % H, bb = bh / H;
    const int t0 = n * CH, c0 = cg * CW;
    const size_t cbase = (size_t)bh * nch + n;
    auto f = [](uint16_t x) { return __uint_as_float((uint32_t)x << 16); };
    const uint16_t* q = static_cast<const uint16_t*>(io.q);
    const uint16_t* k = static_cast<const uint16_t*>(io.k);
    const uint16_t* al = static_cast<const uint16_t*>(io.alpha);
    const uint16_t* b = static_cast<const uint16_t*>(io.b);
    // every global load is issued before the first LDS write, so their latencies overlap
    constexpr int NX = CH * CW / 256, NA = CH * CH / 256;
    uint16_t lq[NX], lk[NX], lb[NX], la[NX];
    float lA[NA], lP[NA];
#pragma unroll
    for (int u = 0; u < NX; ++u) {
        const int x = tid + 256 * u, r = x / CW, i = x % CW;
        const int t = t0 + r;
        const size_t e = (((size_t)bb * T + (t < T ? t : 0)) * H + hh) * DK + c0 + i;
        lq[u] = q[e];
        lk[u] = k[e];
        lb[u] = b[e];
        la[u] = al[e];
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        lA[u] = io.dAm[cbase * CH * CH + tid + 256 * u];
        lP[u] = io.dPm[cbase * CH * CH + tid + 256 * u];
    }
    // this thread's rows p + 8 m of channel i for the elementwise phase: dQ_hat, dE_hat, dK_bar
    const int i = tid % CW, p = tid / CW;
    float gQv[8], gEv[8], gKv[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const size_t ce = (cbase * CH + p + 8 * m) * DK + c0 + i;
        gQv[m] = io.dQh[ce];
        gEv[m] = io.dEh[ce];
        gKv[m] = io.dKb[ce];
    }
    const float dgam_i = io.dgam[cbase * DK + c0 + i];
#pragma unroll
    for (int u = 0; u < NX; ++u) {
        const int x = tid + 256 * u, r = x / CW;
        const bool ok = t0 + r < T;
        qs[x] = ok ? lq[u] : 0;
        ks[x] = ok ? lk[u] : 0;
        bs[x] = ok ? lb[u] : 0;
        G2[x] = ok ? __builtin_amdgcn_logf(f(la[u])) : 0.f;  // rows past the end do not decay
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        dA[tid + 256 * u] = lA[u];
        dPs[tid + 256 * u] = lP[u];
    }
    __syncthreads();
    if (tid < CW) {
        float acc = 0.f;
        for (int r = 0; r < CH; ++r) {
            acc += G2[r * CW + tid];
            G2[r * CW + tid] = acc;
        }
    }
    __syncthreads();
    for (int x = tid; x < CH * CW; x += 256) {
        const int r = x / CW, i = x % CW, I = r / 16;
        const float g = G2[x];
        const float kv = f(ks[x]);
        Kp[x] = kv * __builtin_amdgcn_exp2f(G2[(16 * I + 15) * CW + i] - g);
        const float down = __builtin_amdgcn_exp2f(g - G2[(16 * I) * CW + i]);
        Ep[x] = f(bs[x]) * kv * down;
        Qp[x] = f(qs[x]) * down;
    }
    __syncthreads();

    // Blocks off the diagonal on the matrix cores (fp32 16x16x4): wave w takes row block I = w
    // and both 16-channel tiles. XA, XP of rows in I sum over blocks J < I, Y over blocks I2 > I;
    // each block's product is scaled by its reference factor per (row, channel) and added. The
    // 16 block rows are contracted in 4 passes, lane group g holding rows 4 g .. 4 g + 3.
    {
        const int I = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
        f4 xa[2], xp[2], yy[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) xa[ct] = xp[ct] = yy[ct] = f4{0.f, 0.f, 0.f, 0.f};
        for (int J = 0; J < I; ++J) {
            f4 sa[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
            f4 sp[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ip = 0; ip < 4; ++ip) {
                const int s = 16 * J + 4 * g + ip;
                const float a = dA[(16 * I + l16) * CH + s], pp = dPs[(16 * I + l16) * CH + s];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const float kp = Kp[s * CW + 16 * ct + l16];
                    sa[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, kp, sa[ct], 0, 0, 0);
                    sp[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(pp, kp, sp[ct], 0, 0, 0);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const float ge = G2[(16 * J + 15) * CW + 16 * ct + l16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fJ = __builtin_amdgcn_exp2f(G2[(16 * I + 4 * g + j) * CW + 16 * ct + l16] - ge);
                    xa[ct][j] = fmaf(fJ, sa[ct][j], xa[ct][j]);
                    xp[ct][j] = fmaf(fJ, sp[ct][j], xp[ct][j]);
                }
            }
        }
        for (int I2 = I + 1; I2 < 4; ++I2) {
            f4 sy[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ip = 0; ip < 4; ++ip) {
                const int r2 = 16 * I2 + 4 * g + ip;
                const float a = dA[r2 * CH + 16 * I + l16], pp = dPs[r2 * CH + 16 * I + l16];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    sy[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Ep[r2 * CW + 16 * ct + l16], sy[ct], 0, 0, 0);
                    sy[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(pp, Qp[r2 * CW + 16 * ct + l16], sy[ct], 0, 0, 0);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const float gb = G2[(16 * I2) * CW + 16 * ct + l16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float f = __builtin_amdgcn_exp2f(gb - G2[(16 * I + 4 * g + j) * CW + 16 * ct + l16]);
                    yy[ct][j] = fmaf(f, sy[ct][j], yy[ct][j]);
                }
            }
        }
        __syncthreads();  // every read of Kp, Ep, Qp is done: they take the sums off the diagonal
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int x = (16 * I + 4 * g + j) * CW + 16 * ct + l16;
                Kp[x] = xa[ct][j];
                Ep[x] = xp[ct][j];
                Qp[x] = yy[ct][j];
            }
    }
    __syncthreads();

    const float G63 = G2[(CH - 1) * CW + i];
    float dG[8];
    float kb_sum = 0.f;
    // rows p, p + 8, ..., p + 56 (the row's block I changes every other step)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = p + 8 * m, I = r / 16;
        const float Gr = G2[r * CW + i];
        const float kr = f(ks[r * CW + i]), qr = f(qs[r * CW + i]), br = f(bs[r * CW + i]);
        // XA, XP: the earlier blocks' sums (above), then the diagonal block term by term
        float XA = Kp[r * CW + i], XP = Ep[r * CW + i];
        for (int s = 16 * I; s <= r; ++s) {
            const float w = f(ks[s * CW + i]) * __builtin_amdgcn_exp2f(Gr - G2[s * CW + i]);
            if (s < r) XA = fmaf(dA[r * CH + s], w, XA);
            XP = fmaf(dPs[r * CH + s], w, XP);
        }
        // Y: the later blocks' sums (above), then the diagonal block term by term
        float Y = Qp[r * CW + i];
        for (int r2 = r; r2 < 16 * I + 16; ++r2) {
            const float w = __builtin_amdgcn_exp2f(G2[r2 * CW + i] - Gr);
            const float e2 = f(bs[r2 * CW + i]) * f(ks[r2 * CW + i]);
            float term = dPs[r2 * CH + r] * f(qs[r2 * CW + i]);
            if (r2 > r) term = fmaf(dA[r2 * CH + r], e2, term);
            Y = fmaf(term, w, Y);
        }
        const float eG = __builtin_amdgcn_exp2f(Gr), eK = __builtin_amdgcn_exp2f(G63 - Gr);
        const float gQ = gQv[m], gE = gEv[m], gK = gKv[m];
        const float Et = br * kr;
        const float dEt = fmaf(gE, eG, XA);
        const float dqv = fmaf(gQ, eG, XP);
        const float dkv = fmaf(gK, eK, Y) + br * dEt;
        const float dbv = kr * dEt;
        dG[m] = gQ * qr * eG + gE * Et * eG - gK * kr * eK + Et * XA + qr * XP - kr * Y;
        kb_sum = fmaf(gK, kr * eK, kb_sum);
        const int t = t0 + r;
        if (t < T) {
            const size_t e = (((size_t)bb * T + t) * H + hh) * DK + c0 + i;
            io.dq[e] = dqv;
            io.dk[e] = dkv;
            io.db[e] = dbv;
        }
    }
    red[tid] = kb_sum;
    __syncthreads();  // every read of Kp, Ep, Qp is done
#pragma unroll
    for (int m = 0; m < 8; ++m) Kp[(p + 8 * m) * CW + i] = dG[m];
    __syncthreads();
    // dlog(alpha)_r = sum_{r2 >= r} dG_r2, the last row also carrying the gamma and K_bar terms;
    // thread (i, p) sums rows 8 p .. 8 p + 7, then adds the sums of the segments below it.
    // alpha_r = 2^(G_r - G_{r-1}).
    float seg = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) seg += Kp[(8 * p + u) * CW + i];
    float extra = dgam_i * __builtin_amdgcn_exp2f(G63);
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) extra += red[pp * CW + i];
    __syncthreads();  // every read of red is done
    red[p * CW + i] = seg;
    __syncthreads();
    float acc = extra;
    for (int pp = 7; pp > p; --pp) acc += red[pp * CW + i];
#pragma unroll
    for (int u = 7; u >= 0; --u) {
        const int r = 8 * p + u;
        acc += Kp[r * CW + i];
        const int t = t0 + r;
        if (t < T) {
            const float a = __builtin_amdgcn_exp2f(G2[r * CW + i] - (r ? G2[(r - 1) * CW + i] : 0.f));
            io.dalpha[(((size_t)bb * T + t) * H + hh) * DK + c0 + i] = acc / a;
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
    hipLaunchKernelGGL((bwd_key_kernel<DK>), dim3(BH * nch * (DK / 32)), dim3(256), 0, st, kio);
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
