#pragma once
// chunk_split_kernels.h -- chunkwise (C = 64) Gated DeltaNet-2 prefill as two kernels on gfx950.
//
// Same method and arithmetic as chunk.hip [page "NVIDIA представила Gated DeltaNet-2 с
// канал-wise гейтами …", paragraph "Реализация": chunkwise WY form, C = 64, cumulative
// channel-wise decay absorbed into the rank-1 factors], split where the dependence on the
// state begins:
//
//   prep   one workgroup per (b, h, chunk), all independent. Gate prep, Gram blocks and the UT
//          inverse, as in chunk.hip phases A-E; it writes the chunk's state-free operands to a
//          workspace blob: Q_hat, -E_hat (token-major), K_bar^T, P, T (fp16 for bf16 inputs)
//          and gamma_last (fp32).
//   chain  one workgroup per (b, h, 64 value columns), walking the chunks in order. The blob of
//          chunk n+1 and its v, w rows are copied straight into LDS (global_load_lds, no
//          registers) while chunk n is processed, so the chain waves hold little more than the
//          fp32 state and their MFMA operands:
//              D' = U - E_hat S,  Delta = T D',  O^T = S^T Q_hat^T + Delta^T P^T,
//              S <- Diag(gamma_last) S + K_bar^T Delta.
//
// The blob's byte layout equals the chain kernel's LDS layout (with its row padding), so the
// copy is a flat 16-byte-per-lane stream. The host walks the sequence in ranges of chunks
// through a workspace ring (prep of a range, then chain of the range, the state carried in
// S_out), so the ring can be sized to stay in the Infinity Cache.
#include "chunk_blob.h"
#include "kernels.h"

namespace gdn2 {

namespace {

using namespace chunk;

// Eight elements c0..c0+7 (c0 a multiple of 8) of row r of E_hat or Q_hat to the blob: two
// 8-byte stores for fp16 (the two 4-element units land where en() puts them), two 16-byte
// stores for fp32.
template <typename BL, typename E>
__device__ __forceinline__ void store8_units(E* base, int r, int c0, const float* x) {
    if constexpr (sizeof(E) == 2) {
        h4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = (_Float16)x[i];
            b[i] = (_Float16)x[i + 4];
        }
        *reinterpret_cast<h4*>(base + BL::en(r, c0)) = a;
        *reinterpret_cast<h4*>(base + BL::en(r, c0 + 4)) = b;
    } else {
        reinterpret_cast<float4*>(base + BL::en(r, c0))[0] = make_float4(x[0], x[1], x[2], x[3]);
        reinterpret_cast<float4*>(base + BL::en(r, c0 + 4))[0] = make_float4(x[4], x[5], x[6], x[7]);
    }
}


// Scheduling hint for a run of P products that each read one LDS operand fragment: issue the
// first LA reads, then alternate MPR products (those sharing one read operand) and one read, so
// every matrix-core instruction finds its operand already loaded.
template <int P, int LA = 4, int MPR = 1>
__device__ __forceinline__ void lookahead_schedule() {
    constexpr int la = P < LA ? P : LA;
    __builtin_amdgcn_sched_group_barrier(0x100, la, 0);
#pragma unroll
    for (int i = 0; i < P - la; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, la * MPR, 0);
}

// ------------------------------------------------------------------------------------------
// prep: one (b, h, chunk)
template <int DK, bool F16>
struct PrepSmem {
    using E = typename Prec<F16>::E;
    using BL = Blob<DK, F16>;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int CHP = BL::CHP;
    static constexpr int AP = CH + 4;                   // row stride of A (padded: fragment reads)
    static constexpr int oTot = 0;                      // float [4][DK]
    static constexpr int oX = oTot + 4 * DK * 4;        // float [4][DK]
    static constexpr int oTab = oX + 4 * DK * 4;        // float [kTabs][DK]
    static constexpr int oOut = oTab + kTabs * DK * 4;  // K_bar^T, T (as in the blob), then P
    static constexpr int oKbT = oOut;
    static constexpr int oTm = oKbT + DK * CHP * ES;
    static constexpr int oP = oTm + BL::TPE * ES;
    static constexpr int out1Bytes = BL::oGC - BL::oKbT;  // K_bar^T and T
    static constexpr int outBytes = out1Bytes + BL::TPE * ES;
    static constexpr int KTP = DK + Prec<F16>::kPad;    // 16-byte rows for 16-byte accesses
    static constexpr int oKt = oOut + outBytes;         // E [48][KTP]
    static constexpr int oA = oKt + 48 * KTP * ES;      // E [64][AP] A below the diagonal
    // float [4][ADS] diagonal blocks of A^T, each [16][16]; the block stride is 4 floats more than
    // 256 so that the four 16-lane groups reading four blocks at once hit different banks
    static constexpr int ADS = 260;
    static constexpr int oAd = oA + CH * AP * ES;
    static constexpr int bytes = oAd + 4 * ADS * 4;
    static_assert(BL::oTm - BL::oKbT == DK * CHP * ES && out1Bytes == DK * CHP * ES + BL::TPE * ES, "layout");
    // two workgroups per CU for fp16 blocks up to d = 128 and fp32 blocks of d = 32; one for fp16
    // at d = 256 (its block alone is 110 KB) and fp32 at d = 64 and 128
    static_assert(bytes <= ((F16 ? DK <= 128 : DK <= 32) ? 80 : 160) * 1024, "prep LDS budget");
};

// PRO (prologue): bit 0, q and k are L2-normalised over d_k per token here; bit 1, alpha and b
// (or beta) arrive as pre-activations: log2 alpha = log2 sigma(x), b = sigma(x).
// VAR: packed batch (vt); workgroup x = (chunk of the batch) * H + h, grid an upper bound on the
// chunk count; blocks [h][chunk of the batch] with n_count slots per head. Otherwise workgroup
// x = (chunk - n_first) * B*H + b*H + h over equal-length sequences of T tokens.
template <int DK, bool BF16, bool AS, bool BS, int PRO = 0, bool VAR = false>
__global__ void __launch_bounds__(256, 2)
prep_kernel(const void* q, const void* k, const void* alpha, const void* b, int B, int T, int H,
            int n_first, int n_count, char* ws, VarTab vt) {
    constexpr bool F16 = BF16;
    using PR = Prec<F16>;
    using E = typename PR::E;
    using Frag = typename PR::Frag;
    using BL = Blob<DK, F16>;
    using SM = PrepSmem<DK, F16>;
    constexpr int NKS = DK / 32, CPL = DK / 4;

    __shared__ __attribute__((aligned(16))) char smem[SM::bytes];
    float* ldsTot = reinterpret_cast<float*>(smem + SM::oTot);
    float* ldsX = reinterpret_cast<float*>(smem + SM::oX);
    float* tab = reinterpret_cast<float*>(smem + SM::oTab);
    E* KbT = reinterpret_cast<E*>(smem + SM::oKbT);
    E* Pm = reinterpret_cast<E*>(smem + SM::oP);
    E* Tm = reinterpret_cast<E*>(smem + SM::oTm);
    E* Kt = reinterpret_cast<E*>(smem + SM::oKt);
    E* A16 = reinterpret_cast<E*>(smem + SM::oA);
    float* AdT = reinterpret_cast<float*>(smem + SM::oAd);

    constexpr bool L2N = (PRO & 1) != 0, GL = (PRO & 2) != 0;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    // this workgroup's block slot (bh, nc), the chunk's index n in its sequence, the sequence's
    // first token row tbase and its length Tq
    int bh, nc, n, Tq;
    long tbase;
    if constexpr (VAR) {
        bh = blockIdx.x % H;
        nc = blockIdx.x / H;
        if (nc >= vt.coff[vt.n]) return;
        const int lo = varlen_seq_of(vt, nc);
        n = nc - vt.coff[lo];
        tbase = vt.start[lo];
        Tq = vt.len[lo];
    } else {
        const int BH = B * H;
        bh = blockIdx.x % BH;
        // last chunk first: the blocks written last, those the chain reads first, are then the
        // ones most likely still in the Infinity Cache when the chain starts
        nc = n_count - 1 - (int)(blockIdx.x / BH);
        n = n_first + nc;
        tbase = (long)(bh / H) * T;
        Tq = T;
    }
    const int hh = bh % H;
    const int t0 = n * CH;
    char* blob = ws + ((size_t)bh * n_count + nc) * BL::bytes;
    const int I = wv, r = 16 * I + l16;

    for (int idx = threadIdx.x; idx < CH * CH; idx += blockDim.x) {
        const int rr = idx / CH, cc = idx % CH;
        if ((cc >> 4) > (rr >> 4) && (!F16 || cc < (rr < 32 ? 32 : 64))) {  // stored blocks only
            Pm[BL::tp(rr, cc)] = (E)0.f;
            Tm[BL::tp(rr, cc)] = (E)0.f;
        }
    }

    // ---- A: inputs of this lane's row, log2-decay and its in-block scan ----
    const int t = t0 + r;
    const bool valid = t < Tq;
    const long tok = (tbase + (valid ? t : 0)) * H + hh;
    // All loads are issued before any is used, unconditionally (rows past the end read row 0 of
    // the sequence and are replaced at their first use): alpha first (the scan needs it at once),
    // then q, k, b. vmcnt counts in issue order, so waiting for alpha leaves the rest in flight.
    Raw8<BF16> rq[NKS], rk[NKS], rb[NKS], ra[NKS];
    float lg[CPL];
    float ras_raw = 1.f, rbs_raw = 0.f;
    if constexpr (AS) {
        ras_raw = load_one<BF16>(alpha, tok);
    } else {
#pragma unroll
        for (int s = 0; s < NKS; ++s) ra[s] = gload8<BF16>(alpha, tok * DK + 32 * s + 8 * g);
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const int c0 = 32 * s + 8 * g;
        rq[s] = gload8<BF16>(q, tok * DK + c0);
        rk[s] = gload8<BF16>(k, tok * DK + c0);
        if constexpr (!BS) rb[s] = gload8<BF16>(b, tok * DK + c0);
    }
    if constexpr (BS) rbs_raw = load_one<BF16>(b, tok);
    // keep every load above ahead of the scan: no load may be moved below this point
    asm volatile("" ::: "memory");
    if constexpr (!AS) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) unpack8<BF16>(keep_or<BF16>(ra[s], valid, GL ? INFINITY : 1.f), &lg[8 * s]);
    }
    if constexpr (AS) {
        float x1 = GL ? (valid ? lg2_sigmoid(ras_raw) : 0.f) : lg2(valid ? ras_raw : 1.f);
        x1 += row_shr<1>(x1);
        x1 += row_shr<2>(x1);
        x1 += row_shr<4>(x1);
        x1 += row_shr<8>(x1);
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] = x1;
    } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] = GL ? lg2_sigmoid(lg[e]) : lg2(lg[e]);
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] += row_shr<1>(lg[e]);
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] += row_shr<2>(lg[e]);
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] += row_shr<4>(lg[e]);
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] += row_shr<8>(lg[e]);
    }
    if (l16 == 15 || l16 == 7) {
        float* dst = (l16 == 15 ? ldsTot : ldsX) + I * DK;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            float4* p = reinterpret_cast<float4*>(dst + 32 * s + 8 * g);
            p[0] = make_float4(lg[8 * s], lg[8 * s + 1], lg[8 * s + 2], lg[8 * s + 3]);
            p[1] = make_float4(lg[8 * s + 4], lg[8 * s + 5], lg[8 * s + 6], lg[8 * s + 7]);
        }
    }
    lds_barrier();

    // ---- decay tables (see chunk_common.h) ----
    {
        constexpr int TPC = 256 / DK;
        const int c = threadIdx.x % DK, part = threadIdx.x / DK;
        float tot[4], X[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            tot[J] = ldsTot[J * DK + c];
            X[J] = ldsX[J * DK + c];
        }
        const float G[5] = {0.f, tot[0], tot[0] + tot[1], tot[0] + tot[1] + tot[2],
                            tot[0] + tot[1] + tot[2] + tot[3]};
        float e[kTabs];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            e[J] = X[J];
            e[4 + J] = G[J];
            e[8 + J] = tot[J] - X[J];
            e[12 + J] = G[4] - G[J + 1];
        }
        e[16] = G[4];
        e[17] = tot[1];
        e[18] = tot[1] + tot[2];
        e[19] = tot[2];
#pragma unroll
        for (int tt = 0; tt < kTabs; ++tt)
            if (tt % TPC == part) tab[tt * DK + c] = ex2(e[tt]);
    }
    lds_barrier();

    // ---- B: factors; Q_hat and -E_hat straight to the blob; diagonal Gram blocks ----
    // Prologue: 1 / |q| and 1 / |k| of this lane's row (the row's channels are spread over the
    // four lane groups: lanes l16, l16 + 16, l16 + 32, l16 + 48).
    float nq = 1.f, nk = 1.f;
    if constexpr (L2N) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            float qx[8], kx[8];
            unpack8<BF16>(keep_or<BF16>(rq[s], valid, 0.f), qx);
            unpack8<BF16>(keep_or<BF16>(rk[s], valid, 0.f), kx);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sq = fmaf(qx[i], qx[i], sq);
                sk = fmaf(kx[i], kx[i], sk);
            }
        }
        sq += __shfl_xor(sq, 16);
        sk += __shfl_xor(sk, 16);
        sq += __shfl_xor(sq, 32);
        sk += __shfl_xor(sk, 32);
        nq = 1.f / fmaxf(sqrtf(sq), 1e-12f);
        nk = 1.f / fmaxf(sqrtf(sk), 1e-12f);
    }
    // q, k (normalised) and b of 8 channels of this lane's row, for 32-channel step s
    auto row_gates = [&](int s, float* qx, float* kx, float* bx) {
        if constexpr (L2N) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qx[i] *= nq;
                kx[i] *= nk;
            }
        }
        if constexpr (BS) {
            const float be = GL ? sigmoidf_(rbs_raw) : rbs_raw;
#pragma unroll
            for (int i = 0; i < 8; ++i) bx[i] = valid ? be : 0.f;
        } else {
            unpack8<BF16>(keep_or<BF16>(rb[s], valid, GL ? -INFINITY : 0.f), bx);
            if constexpr (GL) {
#pragma unroll
                for (int i = 0; i < 8; ++i) bx[i] = sigmoidf_(bx[i]);
            }
        }
    };
    float er[CPL], qr[CPL];
    {
        f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
        E* bQh = reinterpret_cast<E*>(blob + BL::oQh);
        E* bEn = reinterpret_cast<E*>(blob + BL::oEn);
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int c0 = 32 * s + 8 * g;
            float qx[8], kx[8], bx[8], X8[8], fX[8], fG[8], fTX[8], fCG[8];
            unpack8<BF16>(keep_or<BF16>(rq[s], valid, 0.f), qx);
            unpack8<BF16>(keep_or<BF16>(rk[s], valid, 0.f), kx);
            row_gates(s, qx, kx, bx);
            lds_read8f(ldsX + I * DK + c0, X8);
            lds_read8f(tab + (0 + I) * DK + c0, fX);
            lds_read8f(tab + (4 + I) * DK + c0, fG);
            lds_read8f(tab + (8 + I) * DK + c0, fTX);
            lds_read8f(tab + (12 + I) * DK + c0, fCG);
            float em[8], qm[8], km[8], qh[8], en[8], kt[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float d = lg[8 * s + i] - X8[i];
                const float fm = ex2(d), fmi = ex2(-d);
                const float bk = bx[i] * kx[i];
                em[i] = bk * fm;
                qm[i] = qx[i] * fm;
                km[i] = kx[i] * fmi;
                const float fl = fm * fX[i];
                er[8 * s + i] = bk * fl;
                qr[8 * s + i] = qx[i] * fl;
                const float gam = fl * fG[i];
                qh[i] = qx[i] * gam;
                en[i] = -(bk * gam);
                kt[i] = km[i] * fTX[i];
                KbT[BL::kbt(c0 + i, r)] = (E)(kt[i] * fCG[i]);
            }
            {
                const Frag kmf = PR::make(km);
                PR::mma(accA, PR::make(em), kmf);
                PR::mma(accP, PR::make(qm), kmf);
            }
            store8_units<BL>(bQh, r, c0, qh);
            store8_units<BL>(bEn, r, c0, en);
            if (I < 3) PR::store8(&Kt[r * SM::KTP + c0], kt);
        }
        bool finite = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) finite = finite && __builtin_isfinite(accA[j]) && __builtin_isfinite(accP[j]);
        if (F16 && !__all(finite)) {
            // Strong decay inside the block: redo the diagonal block with bf16 hi/lo operands.
            accA = f4{0.f, 0.f, 0.f, 0.f};
            accP = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int c0 = 32 * s + 8 * g;
                float qx[8], kx[8], bx[8], X8[8], em[8], qm[8], km[8];
                unpack8<BF16>(keep_or<BF16>(rq[s], valid, 0.f), qx);
                unpack8<BF16>(keep_or<BF16>(rk[s], valid, 0.f), kx);
                row_gates(s, qx, kx, bx);
                lds_read8f(ldsX + I * DK + c0, X8);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float d = lg[8 * s + i] - X8[i];
                    const float fm = ex2(d);
                    em[i] = bx[i] * kx[i] * fm;
                    qm[i] = qx[i] * fm;
                    km[i] = kx[i] * ex2(-d);
                }
                PR::mma_wide(accA, em, km);
                PR::mma_wide(accP, qm, km);
            }
        }
        float4 at;
        at.x = (4 * g + 0) > l16 ? accA[0] : 0.f;
        at.y = (4 * g + 1) > l16 ? accA[1] : 0.f;
        at.z = (4 * g + 2) > l16 ? accA[2] : 0.f;
        at.w = (4 * g + 3) > l16 ? accA[3] : 0.f;
        *reinterpret_cast<float4*>(AdT + I * SM::ADS + l16 * 16 + 4 * g) = at;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 4 * g + j;
            Pm[BL::tp(16 * I + rr, 16 * I + l16)] = (E)(rr >= l16 ? accP[j] : 0.f);
        }
    }
    lds_barrier();

    // ---- C: Gram blocks below the diagonal; T_II ----
    // Wave I computes the blocks (I, J < I) of A and P together, so that their LDS reads and
    // products interleave. Non-adjacent blocks use the row factors times exp2(G_I - G_{J+1})
    // (tables 17..19).
    auto gram_blocks = [&](auto nb_c, const float* c0tab, const float* c1tab) {
        constexpr int NB = decltype(nb_c)::value;
        f4 accA[NB], accP[NB];
#pragma unroll
        for (int J = 0; J < NB; ++J) accA[J] = accP[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int c0 = 32 * s + 8 * g;
            float c8[2][8];
            if constexpr (NB >= 2) lds_read8f(c0tab + c0, c8[0]);
            if constexpr (NB >= 3) lds_read8f(c1tab + c0, c8[1]);
            Frag kf[NB];
#pragma unroll
            for (int J = 0; J < NB; ++J) kf[J] = PR::lds8(Kt + (16 * J + l16) * SM::KTP + c0);
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                float ea[8], qa[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float f = (J == NB - 1) ? 1.f : c8[J][i];
                    ea[i] = er[8 * s + i] * f;
                    qa[i] = qr[8 * s + i] * f;
                }
                PR::mma(accA[J], PR::make(ea), kf[J]);
                PR::mma(accP[J], PR::make(qa), kf[J]);
            }
        }
#pragma unroll
        for (int J = 0; J < NB; ++J) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 16 * I + 4 * g + j;
                A16[rr * SM::AP + 16 * J + l16] = (E)accA[J][j];
                Pm[BL::tp(rr, 16 * J + l16)] = (E)accP[J][j];
            }
        }
    };
    if (wv == 1) {
        gram_blocks(std::integral_constant<int, 1>{}, nullptr, nullptr);
    } else if (wv == 2) {
        gram_blocks(std::integral_constant<int, 2>{}, tab + 17 * DK, nullptr);
    } else if (wv == 3) {
        gram_blocks(std::integral_constant<int, 3>{}, tab + 18 * DK, tab + 19 * DK);
    }
    if (wv == 0) {
        // T_II = (I + A_II)^-1 for the four diagonal blocks, right-looking, by the wave that
        // has no Gram block above: lane group g solves block g, lane l16 owns column l16.
        const int Ib = g;
        float acc[16], tc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = 0.f;
        const float4* Ab4 = reinterpret_cast<const float4*>(AdT + Ib * SM::ADS);
        float4 cur[4], nxt[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) cur[q4] = Ab4[q4];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m + 1 < 16) {
#pragma unroll
                for (int q4 = (m + 2) / 4; q4 < 4; ++q4) nxt[q4] = Ab4[(m + 1) * 4 + q4];
            }
            const float tm = m < l16 ? 0.f : (m == l16 ? 1.f : -acc[m]);
            tc[m] = tm;
#pragma unroll
            for (int q4 = (m + 1) / 4; q4 < 4; ++q4) {
                const float av[4] = {cur[q4].x, cur[q4].y, cur[q4].z, cur[q4].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * q4 + i > m) acc[4 * q4 + i] = fmaf(av[i], tm, acc[4 * q4 + i]);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) Tm[BL::tp(16 * Ib + m, 16 * Ib + l16)] = (E)tc[m];
    }
    lds_barrier();

    // ---- D: T10 = -T11 A10 T00 and T32 = -T33 A32 T22 ----
    if (wv == 1 || wv == 3) {
        const int Ib = wv, Jb = wv - 1;
        float af[8], bf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = (float)A16[(16 * Ib + l16) * SM::AP + 16 * Jb + 4 * g + i];
            bf[i] = (float)Tm[BL::tp(16 * Jb + 4 * g + i, 16 * Jb + l16)];
            af[i + 4] = bf[i + 4] = 0.f;
        }
        f4 X = {0.f, 0.f, 0.f, 0.f};
        PR::mma(X, PR::make(af), PR::make(bf));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = (float)Tm[BL::tp(16 * Ib + l16, 16 * Ib + 4 * g + i)];
            bf[i] = X[i];
        }
        f4 Y = {0.f, 0.f, 0.f, 0.f};
        PR::mma(Y, PR::make(af), PR::make(bf));
#pragma unroll
        for (int j = 0; j < 4; ++j) Tm[BL::tp(16 * Ib + 4 * g + j, 16 * Jb + l16)] = (E)(-Y[j]);
    }
    lds_barrier();

    // ---- E: T[32:, :32] = -T[32:, 32:] A[32:, :32] T[:32, :32] ----
    if (wv < 2) {
        const int Jb = wv;
        f4 Yt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int Ib = 2 + u;
            const E* ar = &A16[(16 * Ib + l16) * SM::AP];
            float bf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) bf[i] = (float)Tm[BL::tp(kap(g, i), 16 * Jb + l16)];
            Yt[u] = f4{0.f, 0.f, 0.f, 0.f};
            PR::mma(Yt[u], PR::lds_pair(ar + 4 * g, ar + 16 + 4 * g), PR::make(bf));
        }
        float yb[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            yb[i] = Yt[0][i];
            yb[i + 4] = Yt[1][i];
        }
        const Frag yf = PR::make(yb);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int Ib = 2 + u;
            const int rw = 16 * Ib + l16;
            f4 Z = {0.f, 0.f, 0.f, 0.f};
            PR::mma(Z, PR::lds_pair(Tm + BL::tp(rw, 32 + 4 * g), Tm + BL::tp(rw, 48 + 4 * g)), yf);
#pragma unroll
            for (int j = 0; j < 4; ++j) Tm[BL::tp(16 * Ib + 4 * g + j, 16 * Jb + l16)] = (E)(-Z[j]);
        }
    }
    lds_barrier();

    // ---- out: K_bar^T and T (contiguous in LDS and in the blob), P, gamma_last ----
    {
        // (256 threads; every LDS read is issued before the stores)
        const int tid = threadIdx.x;
        constexpr int N1 = SM::out1Bytes / 16, NP = BL::TPE * (int)sizeof(E) / 16;
        constexpr int J1 = (N1 + 255) / 256, JP = (NP + 255) / 256;
        const uint4* src = reinterpret_cast<const uint4*>(smem + SM::oOut);
        const uint4* srcP = reinterpret_cast<const uint4*>(smem + SM::oP);
        uint4 v1[J1], vp[JP];
#pragma unroll
        for (int j = 0; j < J1; ++j) v1[j] = src[min(tid + 256 * j, N1 - 1)];
#pragma unroll
        for (int j = 0; j < JP; ++j) vp[j] = srcP[min(tid + 256 * j, NP - 1)];
        // stores through resources bounded by the regions: lanes past the end store nothing
        const auto rs1 = make_rsrc(blob + BL::oKbT, N1 * 16);
        const auto rsP = make_rsrc(blob + BL::oP, NP * 16);
#pragma unroll
        for (int j = 0; j < J1; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&v1[j]), rs1,
                                                   16 * (tid + 256 * j), 0, 0);
#pragma unroll
        for (int j = 0; j < JP; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&vp[j]), rsP,
                                                   16 * (tid + 256 * j), 0, 0);
        float* gc = reinterpret_cast<float*>(blob + BL::oGC);
        static_assert(DK <= 256, "one gamma_last element per thread");
        if (tid < DK) gc[tid] = tab[16 * DK + tid];
        if constexpr (BS) {
            if (g == 0) reinterpret_cast<float*>(blob + BL::oBeta)[r] = valid ? (GL ? sigmoidf_(rbs_raw) : rbs_raw) : 0.f;
        }
    }
}

// ------------------------------------------------------------------------------------------
// chain: one (b, h, value tile), chunks n_first .. n_first + n_count - 1
// Chain kernel shape: each chain wave owns NT 16-column state tiles, which share every operand
// read from LDS; the copy waves stream the next chunk's block.
constexpr int kChainNT = 1;
constexpr int kChainThreads = 2 * (kChainNT == 1 ? 4 : 2) * 64;

// SMALL: the state-only pass of a segmented sequence (no saves). It copies only the block's
// prefix, into one buffer, so its workgroups take under 80 KB of LDS and two share a CU: its grid
// (segments x heads x state and transition tiles) is larger than the chip, and a second
// workgroup on the CU covers the copy that the one buffer leaves exposed.
template <int DK, int DVT, bool F16, bool SMALL = false>
struct ChainSmem {
    using BL = Blob<DK, F16>;
    static constexpr int NT = kChainNT;
    static constexpr int NWC = DVT / (16 * NT);                 // chain waves
    static constexpr int CW0 = NT == 1 ? 4 : 2;                 // first copy wave = copy waves
    static constexpr int VWB = CH * 16 * NT * (F16 ? 2 : 4);  // one of v, w: 64 rows x 16 NT columns
    // fp32 at d = 128: the v, w slots do not fit beside the 135 KB block, so the chain waves load
    // their v, w straight into registers instead
    static constexpr bool VWREG = !F16 && DK == 128;
    // Two block buffers (the copy of chunk n + 1 overlaps chunk n) when they fit; at d = 256 one
    // block is 110 KB, so there is one buffer, the copy follows the chunk, and the chain waves
    // make it themselves: no copy waves, so each chain wave has a SIMD and its 512 registers.
    static constexpr int BUF = SMALL ? (BL::stateBytes + 255) / 256 * 256 : BL::bytes;
    static constexpr bool ONEBUF = SMALL || 2 * BL::bytes + (VWREG ? 0 : NWC * 2 * VWB) > 160 * 1024;
    static constexpr int threads = ONEBUF ? NWC * 64 : kChainThreads;
    static_assert(ONEBUF || threads == 2 * CW0 * 64, "wave layout");
    static constexpr int oBuf0 = 0;
    static constexpr int oBuf1 = ONEBUF ? 0 : BUF;
    static constexpr int oVW = (ONEBUF ? 1 : 2) * BUF;          // per chain wave: v then w
    static constexpr int bytes = oVW + (VWREG ? 16 : NWC * 2 * VWB);
    static constexpr int min_blocks = (SMALL && bytes <= 80 * 1024) ? 2 : 1;
    static constexpr bool fits = bytes <= 160 * 1024 && NWC >= 1 && NWC <= CW0;
};

// Chain waves 0..NWC-1 hold the state; copy waves CW0..2 CW0-1 stream the next chunk's block into
// LDS while the chain waves work on the current one (one wave per SIMD when NT = 2). Each chain
// wave copies its own v, w columns into a private LDS slot, one chunk ahead, so no barrier guards
// them.
// Where one chain launch reads and writes the state, and which chunks each workgroup runs.
// Workgroup (seg, b·h, tile) runs chunks [first + seg·seg_len, min(first + (seg+1)·seg_len, end))
// of its sequence; the block of chunk n sits in ring slot n - first.
struct ChainIO {
    const void* v;
    const void* w;
    float* o;
    const char* ws;  // blocks [b·h][ring]
    int ring, first, end, seg_len, nseg;
    int B, T, H, DV;
    const float* S_in;  // initial state of (bh, seg): S_in + bh·in_bh + seg·in_seg, rows of in_ld
    long in_bh, in_seg;
    int in_ld;
    float* S_out;  // final state: S_out + bh·out_bh + seg·out_seg, rows of out_ld
    long out_bh, out_seg;
    int out_ld;
    int out_last;  // only the last segment writes S_out
    int phi_tiles = 0;  // transition tiles (over d_k) after the value tiles, state-only pass
    // Saves for the backward pass (a single sequential pass, no segments): the state at the start of every
    // chunk (fp16: the precision its readers take it in as matrix-core operands),
    // S_save + ((bh * save_nch) + chunk) * DK * DV; D' and Delta rows, [B, T, H, DV] fp16
    uint16_t* S_save = nullptr;
    int save_nch = 0;
    uint16_t* Dp_save = nullptr;  // fp16 bits
    uint16_t* Dl_save = nullptr;
    // Packed batch (chain_kernel's VAR): workgroup (b·h, tile) runs every chunk of sequence b, the
    // blocks [h][chunk of the batch] with `ring` slots per head; B counts the sequences.
    VarTab var{};
};

// STATE = true: the state recurrence alone, for the segment transitions of a long sequence. Tiles
// below DV / DVT run it from a zero state with the true U (their final state is the segment's
// inhomogeneous part Psi); tiles above run it with U = 0 from the identity on their columns (the
// transition Phi). No o, and only the block prefix the recurrence reads is copied.
// SAVE (for the backward): also write the start state of every chunk and the rows of D' and
// Delta (ChainIO's save fields); with STATE the backward's own recomputation, without it a
// forward that computes o as well and leaves the backward nothing to recompute. Saving keeps the
// state operands unscaled (the saved fp16 values are read as they are).
// WSIG: w arrives as pre-activations (the prologue's gate logits); U = sigma(w) v.
// VAR: packed batch (ChainIO::var); a sequence without tokens only carries S_in to S_out.
template <int DK, int DVT, bool BF16, bool BS, bool STATE, bool SAVE = false, bool WSIG = false,
          bool VAR = false>
__global__ void __launch_bounds__((ChainSmem<DK, DVT, BF16, STATE && !SAVE>::threads),
                                  (ChainSmem<DK, DVT, BF16, STATE && !SAVE>::min_blocks))
chain_kernel(const ChainIO io) {
    constexpr bool F16 = BF16;
    using PR = Prec<F16>;
    using E = typename PR::E;
    using Frag = typename PR::Frag;
    using BL = Blob<DK, F16>;
    using SM = ChainSmem<DK, DVT, F16, STATE && !SAVE>;
    static_assert(SM::fits, "chain LDS budget or wave layout");
    constexpr int NT = SM::NT, NWC = SM::NWC, CW0 = SM::CW0;
    constexpr int NKS = DK / 32, NMK = DK / 16;
    constexpr int COPY = STATE ? BL::stateBytes : BL::bytes;  // bytes of each block copied to LDS

    // Two arrays: the block buffers and the v/w slots. Separate objects let the compiler see that
    // a v/w copy in flight cannot alias the block reads that follow it, so it does not wait for
    // the copy before them.
    __shared__ __attribute__((aligned(16))) char smem[SM::oVW];
    __shared__ __attribute__((aligned(16))) char svw[SM::bytes - SM::oVW];

    const int T = io.T, H = io.H, DV = io.DV;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int vt = DV / DVT;                  // value tiles
    const int tiles = vt + (STATE ? io.phi_tiles : 0);
    const int BH = io.B * H, BHp = (BH + 7) / 8 * 8;
    const int seg = blockIdx.x / (BHp * tiles);
    const int x = blockIdx.x % (BHp * tiles);
    const int grp = x / (8 * tiles), within = x % (8 * tiles);
    const int tile = within / 8;
    int bh = grp * 8 + (within % 8);
    if (bh >= BH || seg >= io.nseg) return;
    // packed batch: the workgroups take the sequences longest first, so the longest chains start
    // at once and the short ones fill in behind them
    if constexpr (VAR) bh = io.var.perm[bh / H] * H + bh % H;
    const int hh = bh % H;
    // chunks [c_begin, c_end) of this sequence, whose blocks start at `blobs`; the sequence's
    // first token row tbase and its length Tq
    int c_begin, c_end, Tq;
    long tbase;
    const char* blobs;
    size_t save_base;  // chunk slot of the saves (SAVE): chunk n of this sequence is save_base + n
    if constexpr (VAR) {
        const int sq = bh / H, cf = io.var.coff[sq];
        c_begin = 0;
        c_end = io.var.coff[sq + 1] - cf;
        tbase = io.var.start[sq];
        Tq = io.var.len[sq];
        blobs = io.ws + ((size_t)hh * io.ring + cf) * BL::bytes;
        save_base = (size_t)hh * io.ring + cf;
    } else {
        c_begin = io.first + seg * io.seg_len;
        c_end = min(c_begin + io.seg_len, io.end);
        tbase = (long)(bh / H) * T;
        Tq = T;
        blobs = io.ws + ((size_t)bh * io.ring + (c_begin - io.first)) * BL::bytes;
        save_base = (size_t)bh * io.save_nch;
    }
    const int n_count = c_end - c_begin;
    if (!VAR && n_count <= 0) return;
    const bool phi = STATE && tile >= vt;     // transition tile: U = 0, identity start
    const bool chain = wv < NWC;
    const bool copier = !SM::ONEBUF && wv >= CW0;  // one buffer: the chain waves copy
    // this wave's first state column: in v space, or in k space for a transition tile
    const int col0 = (phi ? (tile - vt) : tile) * DVT + (chain ? wv : 0) * 16 * NT;
    float* const o = io.o;
    const void* const v = io.v;
    const void* const w = io.w;
    // o of one chunk's rows as a buffer (rebased per chunk; rows past the end are dropped): byte
    // offset of the chunk's token row l16 at this lane's four columns of tile 0, and the byte
    // stride of one token
    const unsigned o_lane = (((unsigned)l16 * H + hh) * DV + col0 + 4 * g) * 4u;
    const unsigned o_tok = (unsigned)H * DV * 4u;

    f4 Sacc[NT][NMK];
    const float* s_in = io.S_in ? io.S_in + bh * io.in_bh + seg * io.in_seg : nullptr;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * mk + 4 * g + j, col = col0 + 16 * c + l16;
                float x0 = 0.f;
                if (phi) {
                    x0 = row == col ? 1.f : 0.f;
                } else if (chain && s_in) {
                    x0 = s_in[(long)row * io.in_ld + col];
                }
                Sacc[c][mk][j] = x0;
            }

    // fp16 operands (bf16 inputs): the state and each chunk's products are held times sc, a power
    // of two per wave (isc = 1 / sc), so that they stay inside fp16's range whatever the state's
    // magnitude; exact in binary. The state-only pass that saves states for the backward keeps
    // sc = 1 (its saved fp16 values are read unscaled).
    constexpr bool SCALE = F16 && !SAVE;
    static_assert(!SCALE || NT == 1, "the scale is renewed over one 16-column tile per wave");
    int esc = 0;
    float sc = 1.f, isc = 1.f;

    // v and w rows of this wave's columns for one chunk, copied into the wave's LDS slot through
    // buffer resources over the chunk's rows (rebased per chunk, so offsets stay small whatever the
    // sequence length): rows past the sequence end fall outside the buffer and arrive as zeros. A
    // scalar beta comes with the chunk's block instead of w.
    using Raw = typename std::conditional<BF16, uint16_t, uint32_t>::type;
    constexpr int IES = (int)sizeof(Raw);
    constexpr int ROW = 16 * NT;             // elements per slot row
    constexpr int LPR = ROW * IES / 16;      // lanes per slot row in a copy
    constexpr int RPI = 64 / LPR;            // rows per copy instruction
    char* vw_lds = svw + (chain ? wv : 0) * 2 * SM::VWB;
    const Raw* v_l = reinterpret_cast<const Raw*>(vw_lds);
    const Raw* w_l = reinterpret_cast<const Raw*>(vw_lds + SM::VWB);
    auto dma_vw = [&](int n) {
        const __amdgpu_buffer_rsrc_t rs_v = rows_rsrc(v, tbase, (long)n * CH, Tq, (unsigned)(H * DV * IES), CH);
        const __amdgpu_buffer_rsrc_t rs_w = rows_rsrc(BS ? v : w, tbase, (long)n * CH, Tq, (unsigned)(H * DV * IES), CH);
#pragma unroll
        for (int k = 0; k < CH / RPI; ++k) {
            // slot row p holds token row 16 (p / 16) + 4 (p % 4) + (p / 4) % 4, so that the four
            // rows 4 g + j (g = 0..3) read together sit in consecutive slot rows
            const int p = k * RPI + lane / LPR;
            const unsigned row = (unsigned)(16 * (p / 16) + 4 * (p % 4) + (p / 4) % 4);
            const unsigned off = ((row * H + hh) * DV + (unsigned)col0) * IES + (lane % LPR) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_v, (lds_ptr_t)(vw_lds + k * 1024), 16, off, 0, 0, 0);
            if constexpr (!BS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (lds_ptr_t)(vw_lds + SM::VWB + k * 1024), 16, off,
                                                         0, 0, 0);
        }
    };
    // (VWREG) this lane's v, w of a chunk in registers, in the accumulator layout: rows
    // 16 mt + 4 g + j, column col0 + 16 c + l16, through buffer resources over the chunk's rows
    // (rows past the end arrive as zeros)
    Raw vreg[NT][16], wreg[NT][16];
    auto load_vw = [&](int n) {
        if constexpr (SM::VWREG) {
            const __amdgpu_buffer_rsrc_t rs_v = rows_rsrc(v, tbase, (long)n * CH, Tq, (unsigned)(H * DV * IES), CH);
            const __amdgpu_buffer_rsrc_t rs_w = rows_rsrc(BS ? v : w, tbase, (long)n * CH, Tq, (unsigned)(H * DV * IES), CH);
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const unsigned row = (unsigned)(16 * mt + 4 * g + j);
                        const int off = (int)(((row * H + hh) * DV + (unsigned)(col0 + 16 * c + l16)) * IES);
                        vreg[c][4 * mt + j] = (Raw)__builtin_amdgcn_raw_buffer_load_b32(rs_v, off, 0, 0);
                        if constexpr (!BS) wreg[c][4 * mt + j] = (Raw)__builtin_amdgcn_raw_buffer_load_b32(rs_w, off, 0, 0);
                    }
        } else {
            dma_vw(n);
        }
    };
    auto raw_f = [](Raw r) { return BF16 ? __uint_as_float((uint32_t)r << 16) : __uint_as_float((uint32_t)r); };
    // two stacked 16-row accumulator tiles as one operand fragment (the kap() slot order)
    auto stack = [](const f4& lo, const f4& hi) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t[i] = lo[i];
            t[i + 4] = hi[i];
        }
        return PR::make(t);
    };

    // accumulator tiles of 64 token rows x 16 columns ([mt][j]: row 16 mt + 4 g + j, column l16 of
    // tile c) to [B, T, H, DV] fp16 rows of this sequence (their reader takes them as fp16 matrix-core
    // operands); rows past the end are dropped
    int t0_cur = 0;
    auto save_rows = [&](uint16_t* dst, const f4 (&X)[NT][4]) {
        const __amdgpu_buffer_rsrc_t rs = rows_rsrc(dst, tbase, t0_cur, Tq, (unsigned)(H * DV * 2), CH);
        // this lane's byte offset in the chunk's row 4 g, plus a uniform stride per stored row
        const unsigned lb = (((unsigned)(4 * g) * H + hh) * DV + col0 + l16) * 2u;
        const unsigned rstride = (unsigned)(H * DV) * 2u;
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)X[c][mt][j]), rs,
                                                          (int)(lb + (unsigned)(16 * mt + j) * rstride + 32u * c), 0, 0);
    };

    if (n_count > 0) {  // (no copies in flight when there is no chunk to wait for them)
        if (copier) {
            dma_flat(blobs, smem + SM::oBuf0, COPY, wv - CW0, CW0, lane);
            wait_dma();
        } else if (chain && !phi) {
            load_vw(c_begin);
        }
        if constexpr (SM::ONEBUF) {
            dma_flat(blobs, smem + SM::oBuf0, COPY, wv, NWC, lane);
            wait_dma();
        }
    }

    for (int nc = 0; nc < n_count; ++nc) {
        const int n = c_begin + nc;
        const int t0 = n * CH;
        t0_cur = t0;
        char* buf = smem + ((nc & 1) ? SM::oBuf1 : SM::oBuf0);
        const E* Qh = reinterpret_cast<const E*>(buf + BL::oQh);
        const E* En = reinterpret_cast<const E*>(buf + BL::oEn);
        const E* KbT = reinterpret_cast<const E*>(buf + BL::oKbT);
        const E* Pm = reinterpret_cast<const E*>(buf + BL::oP);
        const E* Tm = reinterpret_cast<const E*>(buf + BL::oTm);
        const float* gC = reinterpret_cast<const float*>(buf + BL::oGC);
        const float* betaL = reinterpret_cast<const float*>(buf + BL::oBeta);

        lds_barrier();  // chunk nc's blob is in LDS; the other buffer is free

        if (chain) {
            // D' starts as U = w v, from this wave's slot. Its copy was issued before the previous
            // chunk's 32 NT D', Delta saves (SAVE) and 4 NT o stores (not STATE), so this wait
            // covers it and leaves those stores in flight.
            if (nc == 0 || (STATE && !SAVE)) {
                wait_dma();
            } else {
                wait_vm_but<(SAVE ? 32 * NT : 0) + (STATE ? 0 : 4 * NT)>();
            }
            if constexpr (SAVE) {
                // the state at the start of this chunk, for the backward pass
                const __amdgpu_buffer_rsrc_t rsv = make_rsrc(io.S_save + (save_base + n) * DK * DV, DK * DV * 2u);
                const unsigned sb = ((unsigned)(4 * g) * DV + col0 + l16) * 2u;
#pragma unroll
                for (int c = 0; c < NT; ++c)
#pragma unroll
                    for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                __builtin_bit_cast(uint16_t, (_Float16)Sacc[c][mk][j]), rsv,
                                (int)(sb + (unsigned)(16 * mk + j) * (unsigned)DV * 2u + 32u * c), 0, 0);
            }
            f4 D[NT][4];
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = 16 * mt + 4 * g + j, slot = 16 * mt + 4 * j + g, cl = 16 * c + l16;
                        const Raw wr = SM::VWREG ? wreg[c][4 * mt + j] : w_l[slot * ROW + cl];
                        const Raw vr = SM::VWREG ? vreg[c][4 * mt + j] : v_l[slot * ROW + cl];
                        float ww = BS ? betaL[row] : raw_f(wr);
                        if constexpr (WSIG && !BS) ww = sigmoidf_(ww);
                        D[c][mt][j] = phi ? 0.f : ww * raw_f(vr);
                    }
            if constexpr (SCALE) rescale_state<NMK>(Sacc[0], D[0], esc, sc, isc);
            float4 gcv[NMK];  // gamma_last of this lane's state rows
#pragma unroll
            for (int mk = 0; mk < NMK; ++mk) gcv[mk] = *reinterpret_cast<const float4*>(gC + 16 * mk + 4 * g);
            __builtin_amdgcn_sched_barrier(0);  // keep these reads out of the operand pipeline below
            Frag Sf[NT][NKS];
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int s = 0; s < NKS; ++s) Sf[c][s] = stack(Sacc[c][2 * s], Sacc[c][2 * s + 1]);
            // D' = U - E_hat S ; O^T = S^T Q_hat^T (each operand read feeds all NT tiles)
            f4 O[NT][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int c = 0; c < NT; ++c) O[c][mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const int rw = 16 * mt + l16;
                    const Frag ef = PR::lds_pair(En + BL::en(rw, 32 * s + 4 * g), En + BL::en(rw, 32 * s + 16 + 4 * g));
#pragma unroll
                    for (int c = 0; c < NT; ++c) PR::mma(D[c][mt], ef, Sf[c][s]);
                    if constexpr (!STATE) {
                        const Frag qf =
                            PR::lds_pair(Qh + BL::en(rw, 32 * s + 4 * g), Qh + BL::en(rw, 32 * s + 16 + 4 * g));
#pragma unroll
                        for (int c = 0; c < NT; ++c) PR::mma(O[c][mt], Sf[c][s], qf);
                    }
                }
            }
            if constexpr (F16) lookahead_schedule<(STATE ? 4 : 8) * NKS, 6, NT>();
            // the next chunk's v, w into this wave's slot, now that its reads are long done
            if (nc + 1 < n_count && !phi) load_vw(n + 1);
            if constexpr (SAVE) save_rows(io.Dp_save, D);
            // Delta = T D'
            Frag Df[NT][2];
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) Df[c][s2] = stack(D[c][2 * s2], D[c][2 * s2 + 1]);
            f4 Dl[NT][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int c = 0; c < NT; ++c) Dl[c][mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 <= mt / 2; ++s2) {
                    const int rw = 16 * mt + l16;
                    const Frag tf = PR::lds_pair(Tm + BL::tp(rw, 32 * s2 + 4 * g), Tm + BL::tp(rw, 32 * s2 + 16 + 4 * g));
#pragma unroll
                    for (int c = 0; c < NT; ++c) PR::mma(Dl[c][mt], tf, Df[c][s2]);
                }
            }
            if constexpr (F16) lookahead_schedule<6, 4, NT>();
            if constexpr (SAVE) save_rows(io.Dl_save, Dl);
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) Df[c][s2] = stack(Dl[c][2 * s2], Dl[c][2 * s2 + 1]);
            // O^T += Delta^T P^T and S <- Diag(gamma_last) S + K_bar^T Delta: independent
            // products on one pipelined stream of operand reads
            if constexpr (!STATE) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                    for (int s2 = 0; s2 <= nt / 2; ++s2) {
                        const int rw = 16 * nt + l16;
                        const Frag pf =
                            PR::lds_pair(Pm + BL::tp(rw, 32 * s2 + 4 * g), Pm + BL::tp(rw, 32 * s2 + 16 + 4 * g));
#pragma unroll
                        for (int c = 0; c < NT; ++c) PR::mma(O[c][nt], Df[c][s2], pf);
                    }
                }
            }
#pragma unroll
            for (int mk = 0; mk < NMK; ++mk) {
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    Sacc[c][mk][0] *= gcv[mk].x;
                    Sacc[c][mk][1] *= gcv[mk].y;
                    Sacc[c][mk][2] *= gcv[mk].z;
                    Sacc[c][mk][3] *= gcv[mk].w;
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int rw = 16 * mk + l16;
                    const Frag kf =
                        PR::lds_pair(KbT + BL::kbt(rw, 32 * s2 + 4 * g), KbT + BL::kbt(rw, 32 * s2 + 16 + 4 * g));
#pragma unroll
                    for (int c = 0; c < NT; ++c) PR::mma(Sacc[c][mk], kf, Df[c][s2]);
                }
            }
            if constexpr (F16) lookahead_schedule<(STATE ? 0 : 6) + 2 * NMK, 6, NT>();
            if constexpr (!STATE) {
                // o rows of this chunk: four consecutive columns per lane and tile, one 16-byte
                // store each (always 4 NT stores per chunk; rows past the end are dropped)
                const __amdgpu_buffer_rsrc_t rs_o = rows_rsrc(o, tbase, t0, Tq, o_tok, CH);
                const unsigned op = o_lane;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int c = 0; c < NT; ++c)
                        store4<kStreamStore>(rs_o, op + 16u * nt * o_tok + 64u * c, O[c][nt][0] * isc,
                                             O[c][nt][1] * isc, O[c][nt][2] * isc, O[c][nt][3] * isc);
            }
        } else if (copier && !SM::ONEBUF) {
            // copy waves: the next chunk's blob, then wait for the copies before the next
            // chunk's barrier
            if (nc + 1 < n_count)
                dma_flat(blobs + (size_t)(nc + 1) * BL::bytes, smem + ((nc & 1) ? SM::oBuf0 : SM::oBuf1), COPY,
                         wv - CW0, CW0, lane);
            wait_dma();
        }
        if constexpr (SM::ONEBUF) {
            // one buffer: the next chunk's blob replaces this one once every chain wave is done
            // with it (the barrier at the top of the loop then waits for the copy)
            lds_barrier();
            if (nc + 1 < n_count) dma_flat(blobs + (size_t)(nc + 1) * BL::bytes, smem + SM::oBuf0, COPY, wv, NWC, lane);
            wait_dma();
        }
    }

    if (chain && io.S_out && (!io.out_last || seg == io.nseg - 1)) {
        float* s_out = io.S_out + bh * io.out_bh + seg * io.out_seg + (phi ? DV : 0);
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    s_out[(long)(16 * mk + 4 * g + j) * io.out_ld + col0 + 16 * c + l16] = Sacc[c][mk][j] * isc;
    }
}

// ------------------------------------------------------------------------------------------
// segment scan: S_in[g + 1] = Phi_g S_in[g] + Psi_g, for one (b, h) and 8 state columns, fp32
// psiphi: [b·h][G - 1][DK][DV + DK] (Psi in columns 0..DV-1, Phi in DV..DV+DK-1)
// sseg:   [b·h][G][DK][DV], sseg[·][0] = S0 (or zeros)
template <int DK>
__global__ void __launch_bounds__(256, 1)
scan_kernel(const float* S0, const float* __restrict__ psiphi, float* __restrict__ sseg, int G, int DV) {
    constexpr int CW = 8;           // state columns per workgroup
    constexpr int SETS = 256 / DK;  // column sets per row
    constexpr int CPT = CW / SETS;  // columns per thread
    static_assert(CPT >= 1, "columns per thread");
    __shared__ float cur[DK][CW + 1];
    const int cols = DV / CW;
    const int bh = blockIdx.x / cols, c0 = (blockIdx.x % cols) * CW;
    const int i = threadIdx.x % DK, cb = (threadIdx.x / DK) * CPT;
    const int ld = DV + DK;
    float* out = sseg + (long)bh * G * DK * DV;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        const float x = S0 ? S0[((long)bh * DK + i) * DV + c0 + cb + e] : 0.f;
        cur[i][cb + e] = x;
        out[(long)i * DV + c0 + cb + e] = x;
    }
    __syncthreads();
    for (int gg = 0; gg + 1 < G; ++gg) {
        const float* pp = psiphi + ((long)bh * (G - 1) + gg) * DK * ld + (long)i * ld;
        float acc[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] = pp[c0 + cb + e];
        for (int k = 0; k < DK; k += 4) {
            const float4 f = *reinterpret_cast<const float4*>(pp + DV + k);
#pragma unroll
            for (int e = 0; e < CPT; ++e)
                acc[e] += f.x * cur[k][cb + e] + f.y * cur[k + 1][cb + e] + f.z * cur[k + 2][cb + e] +
                          f.w * cur[k + 3][cb + e];
        }
        __syncthreads();  // every read of cur is done
        out += (long)DK * DV;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            cur[i][cb + e] = acc[e];
            out[(long)i * DV + c0 + cb + e] = acc[e];
        }
        __syncthreads();
    }
}

}  // namespace

}  // namespace gdn2
