// chunk.hip -- chunkwise (C = 64) Gated DeltaNet-2 prefill on gfx950 matrix cores.
//
// Method [page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph
// "Реализация"]: a chunkwise WY form with chunk length 64, the cumulative channel-wise decay
// absorbed into the rank-1 factors. For one chunk of rows r with incoming state S (all per
// key channel, Gamma_r = sum_{s<=r} log alpha_s, gamma = exp(Gamma)):
//     A = strictLower(E_hat K_hat^T), P = lowerIncl(Q_hat K_hat^T)
//         e_hat_r = gamma_r b_r k_r, k_hat_j = k_j / gamma_j, q_hat_r = gamma_r q_r
//     T = (I + A)^-1,  W = T E_hat,  U~ = T (w v)                          (UT transform)
//     Delta = U~ - W S,  O = Q_hat S + P Delta,  S <- Diag(gamma_last) S + K_bar^T Delta
//         k_bar_j = (gamma_last / gamma_j) k_j
// which equals the token-by-token update S_t = (I - k_t (b_t k_t)^T) Diag(alpha_t) S_{t-1}
// + k_t (w_t v_t)^T with o_t = S_t^T q_t [same page, paragraph "Техническая схема"].
//
// Mapping. One workgroup (4 wavefronts) owns one (b, h) and a tile of DVT value columns; the
// columns of S evolve independently given T, E_hat and U, so tiles need no communication. The
// inputs of chunk n+1 are loaded into registers while chunk n is processed. Per chunk:
//   A  wave I takes token rows 16I..16I+15 (lane = row, 8 channels per K-step), converts
//      alpha to log2 and scans it over its 16 rows with row-shift DPP adds; block totals and
//      each block's 8th-row value go to LDS.
//   -  decay tables, once per (block, channel): exp2 of the block references, of the earlier
//      blocks' total G_I, and the factors that link them, so each element needs two exp2.
//   B  factors: Q_hat, -E_hat, K_bar^T, U and block-referenced K~ tiles go to LDS. The diagonal
//      16x16 Gram blocks are formed in registers with factors referenced to the block's 8th
//      row (no factor exceeds the decay of 8 tokens): one fp16 pass when all of the wave's
//      operands fit fp16, else a bf16 hi/lo split (three passes, fp32 exponent range).
//   C  Gram blocks below the diagonal: row side exp2(local), column side
//      exp2(blocktot - local), both <= 1, and for non-adjacent blocks a column side pre-scaled
//      by exp2(G_I - G_{J+1}) <= 1; one fp16 pass. Each wave inverts its 16x16 diagonal block
//      of (I + A) in fp32, right-looking (each finished column updates the rows below).
//   D,E  the 16x16 inverses are merged into the 64x64 T at 32 and 64 rows:
//      T10 = -T11 A10 T00 per 32-row half, then T[32:,:32] = -T[32:,32:] A[32:,:32] T[:32,:32].
//   F  the state chain: each wave owns 16 state columns, held in accumulator registers (fp32)
//      for the whole sequence, and computes D' = U - E_hat S, Delta = T D' (= U~ - W S),
//      O^T = S^T Q_hat^T + Delta^T P^T, S = gamma_last S + K_bar^T Delta. Accumulator tiles feed the next
//      product directly: operand k-slots are chosen to match the accumulator layout (kap
//      below), and the A operands read LDS in the same order.
//
// Precision: with bf16 inputs the products take fp16 operands (fp32 accumulation, fp32 state,
// fp32 o); with fp32 inputs they take fp32 operands (v_mfma_f32_16x16x4_f32).
#include "chunk_common.h"
#include "kernels.h"

namespace gdn2 {

namespace {

using namespace chunk;

// ---- LDS layout ----------------------------------------------------------------------------
template <int DK, int DVT, bool F16>
struct Smem {
    using E = typename Prec<F16>::E;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int PAD = Prec<F16>::kPad;
    static constexpr int DKP = DK + PAD;  // token-major rows over channels
    static constexpr int CHP = CH + PAD;  // rows over 64 tokens
    static constexpr int A32P = CH + 4;   // fp32 A rows
    static constexpr int UP = DVT + 4;    // fp32 U rows
    static constexpr int oTot = 0;                          // float [4][DK]
    static constexpr int oX = oTot + 4 * DK * 4;            // float [4][DK]
    static constexpr int oTab = oX + 4 * DK * 4;            // float [kTabs][DK]
    static constexpr int oQh = oTab + kTabs * DK * 4;       // E [64][DKP]   q_hat
    static constexpr int oEn = oQh + CH * DKP * ES;         // E [64][DKP]   -e_hat
    static constexpr int oKbT = oEn + CH * DKP * ES;        // E [DK][CHP]   k_bar^T
    static constexpr int oP = oKbT + DK * CHP * ES;         // E [64][CHP]   P
    static constexpr int oTm = oP + CH * CHP * ES;          // E [64][CHP]   T
    static constexpr int oKt = oTm + CH * CHP * ES;         // E [48][DKP]   k~ of blocks 0..2
    static constexpr int oKs = oKt + 48 * DKP * ES;         // E [3][16][DKP] k~ of pairs (2,0),(3,0),(3,1)
    static constexpr int oA = oKs + 48 * DKP * ES;          // float [64][A32P] A below the diagonal
    static constexpr int oAd = oA + CH * A32P * 4;          // float [4][16][16] diagonal A^T
    static constexpr int oU = oAd + 4 * 256 * 4;            // float [64][UP] U = w v
    static constexpr int bytes = oU + CH * UP * 4;
    static constexpr bool fits = bytes <= 160 * 1024;
};

template <int DK, int DVT, bool BF16, bool AS, bool BS>
__global__ void __launch_bounds__(256, 1)
chunk_kernel(const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
             const void* __restrict__ alpha, const void* __restrict__ b,
             const void* __restrict__ w, const float* S0, float* __restrict__ o, float* S_out,
             int B, int T, int H, int DV) {
    constexpr bool F16 = BF16;  // bf16 inputs -> fp16 matrix-core operands; fp32 -> fp32
    using PR = Prec<F16>;
    using E = typename PR::E;
    using Frag = typename PR::Frag;
    using SM = Smem<DK, DVT, F16>;
    static_assert(SM::fits, "LDS budget exceeded");
    constexpr int NKS = DK / 32;   // K-steps over channels
    constexpr int NMK = DK / 16;   // 16-row tiles over channels
    constexpr int NWC = DVT / 16;  // waves owning state columns
    constexpr int CPL = DK / 4;    // channels per lane in the token-major layout
    constexpr int NCV = DVT / 4;   // value columns per lane in the token-major layout
    constexpr int DKP = SM::DKP, CHP = SM::CHP, A32P = SM::A32P, UP = SM::UP;

    __shared__ __attribute__((aligned(16))) char smem[SM::bytes];
    float* ldsTot = reinterpret_cast<float*>(smem + SM::oTot);
    float* ldsX = reinterpret_cast<float*>(smem + SM::oX);
    float* tab = reinterpret_cast<float*>(smem + SM::oTab);
    E* Qh = reinterpret_cast<E*>(smem + SM::oQh);
    E* En = reinterpret_cast<E*>(smem + SM::oEn);
    E* KbT = reinterpret_cast<E*>(smem + SM::oKbT);
    E* Pm = reinterpret_cast<E*>(smem + SM::oP);
    E* Tm = reinterpret_cast<E*>(smem + SM::oTm);
    E* Kt = reinterpret_cast<E*>(smem + SM::oKt);
    E* Ks = reinterpret_cast<E*>(smem + SM::oKs);
    float* A32 = reinterpret_cast<float*>(smem + SM::oA);
    float* AdT = reinterpret_cast<float*>(smem + SM::oAd);
    float* U32 = reinterpret_cast<float*>(smem + SM::oU);

    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;

    // Work item. Workgroups are dealt round-robin over the 8 XCDs; x and x + 8 share an XCD,
    // so the value tiles of one (b, h) are placed 8 apart and share q, k, alpha, b in L2.
    const int tiles = DV / DVT;
    const int x = blockIdx.x;
    const int grp = x / (8 * tiles), within = x % (8 * tiles);
    const int tile = within / 8;
    const int bh = grp * 8 + (within % 8);
    if (bh >= B * H) return;  // uniform over the workgroup
    const int hh = bh % H, bb = bh / H;
    const int mycol = tile * DVT + wv * 16 + l16;  // state column owned in the chain
    const bool chain = wv < NWC;
    const int I = wv;              // 16-row block handled in the gate and Gram phases
    const int r = 16 * I + l16;    // chunk row of this lane in those phases

    // Upper-triangle blocks of P and T are zero and never written again.
    for (int idx = threadIdx.x; idx < CH * CH; idx += blockDim.x) {
        const int rr = idx / CH, cc = idx % CH;
        if ((cc >> 4) > (rr >> 4)) {
            Pm[rr * CHP + cc] = (E)0.f;
            Tm[rr * CHP + cc] = (E)0.f;
        }
    }

    // State columns in accumulator layout: Sacc[mk][j] = S[16 mk + 4 g + j][mycol].
    f4 Sacc[NMK];
    const long sbase = (long)bh * DK * DV;
#pragma unroll
    for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sacc[mk][j] = (chain && S0) ? S0[sbase + (long)(16 * mk + 4 * g + j) * DV + mycol] : 0.f;
    int esc = 0;  // the state is held times sc = 2^esc (fp16 operands; see rescale_state)
    float sc = 1.f, isc = 1.f;

    // Inputs of one chunk row for this lane, loaded one chunk ahead. The loads of the next
    // chunk are issued in portions spread over the current one, each as soon as its registers
    // are free (part 0: alpha after the scan; 1: q, v, w after the factors; 2: k and 3: b
    // during the state chain), so the vector-memory queue never backs up into the issuing wave.
    Raw8<BF16> rq[NKS], rk[NKS], rb[NKS], ra[NKS], rv[NCV / 8], rw[NCV / 8];
    float ras = 1.f, rbs = 0.f;
    auto fetch = [&](int n, int part) {
        // loads are unconditional (rows past the end read row 0 of the sequence); the values are
        // replaced at their first use, so the compiler can count the loads in flight exactly
        const int t = n * CH + r;
        const long tok = ((long)bb * T + (t < T ? t : 0)) * H + hh;
        if (part == 0) {
            if constexpr (AS) {
                ras = load_one<BF16>(alpha, tok);
            } else {
#pragma unroll
                for (int s = 0; s < NKS; ++s)
                    ra[s] = gload8<BF16>(alpha, tok * DK + 32 * s + 8 * g);
            }
        } else if (part == 1) {
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                rq[s] = gload8<BF16>(q, tok * DK + 32 * s + 8 * g);
            const int v0 = tile * DVT + g * NCV;
#pragma unroll
            for (int u = 0; u < NCV / 8; ++u) {
                rv[u] = gload8<BF16>(v, tok * DV + v0 + 8 * u);
                if constexpr (!BS) rw[u] = gload8<BF16>(w, tok * DV + v0 + 8 * u);
            }
        } else if (part == 2) {
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                rk[s] = gload8<BF16>(k, tok * DK + 32 * s + 8 * g);
        } else {
            if constexpr (BS) {
                rbs = load_one<BF16>(b, tok);
            } else {
#pragma unroll
                for (int s = 0; s < NKS; ++s)
                    rb[s] = gload8<BF16>(b, tok * DK + 32 * s + 8 * g);
            }
        }
    };

    // o of one chunk's rows as a buffer (rebased per chunk): rows past the end are dropped, so
    // stores need no branch
    const int nch = (T + CH - 1) / CH;
    for (int part = 0; part < 4; ++part) fetch(0, part);
    for (int n = 0; n < nch; ++n) {
        const int t0 = n * CH;
        const int L = min(CH, T - t0);
        const bool vrow = t0 + r < T;  // this lane's row exists

        // ---------------- A: log2-decay and its scan over the block's 16 rows ----------------
        float lg[CPL];
        if constexpr (AS) {
            float x1 = lg2(vrow ? ras : 1.f);
            x1 += row_shr<1>(x1);
            x1 += row_shr<2>(x1);
            x1 += row_shr<4>(x1);
            x1 += row_shr<8>(x1);
#pragma unroll
            for (int e = 0; e < CPL; ++e) lg[e] = x1;
        } else {
#pragma unroll
            for (int s = 0; s < NKS; ++s) unpack8<BF16>(keep_or<BF16>(ra[s], vrow, 1.f), &lg[8 * s]);
#pragma unroll
            for (int e = 0; e < CPL; ++e) lg[e] = lg2(lg[e]);
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

        // ---------------- decay tables, once per (block, channel) ----------------
        const bool more = n + 1 < nch;
        if (more) fetch(n + 1, 0);
        {
            constexpr int TPC = 256 / DK;  // threads per channel
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
            for (int t = 0; t < kTabs; ++t)
                if (t % TPC == part) tab[t * DK + c] = ex2(e[t]);
        }
        lds_barrier();

        // ---------------- B: factors, LDS operand tiles, diagonal Gram blocks ----------------
        Frag erf[NKS], qrf[NKS];  // row-side Gram factors (block-start reference)
        {
            // Diagonal Gram blocks use one fp16 pass; if any operand overflowed fp16 (the
            // accumulators are then not finite) the block is recomputed below with a bf16 hi/lo
            // split.
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int c0 = 32 * s + 8 * g;
                float qx[8], kx[8], bx[8], X8[8], fX[8], fG[8], fTX[8], fCG[8];
                unpack8<BF16>(keep_or<BF16>(rq[s], vrow, 0.f), qx);
                unpack8<BF16>(keep_or<BF16>(rk[s], vrow, 0.f), kx);
                if constexpr (BS) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) bx[i] = vrow ? rbs : 0.f;
                } else {
                    unpack8<BF16>(keep_or<BF16>(rb[s], vrow, 0.f), bx);
                }
                lds_read8f(ldsX + I * DK + c0, X8);
                lds_read8f(tab + (0 + I) * DK + c0, fX);
                lds_read8f(tab + (4 + I) * DK + c0, fG);
                lds_read8f(tab + (8 + I) * DK + c0, fTX);
                lds_read8f(tab + (12 + I) * DK + c0, fCG);
                float em[8], qm[8], km[8], er[8], qr[8], qh[8], en[8], kt[8], kb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float d = lg[8 * s + i] - X8[i];
                    const float fm = ex2(d), fmi = ex2(-d);
                    const float bk = bx[i] * kx[i];
                    em[i] = bk * fm;
                    qm[i] = qx[i] * fm;
                    km[i] = kx[i] * fmi;
                    const float fl = fm * fX[i];
                    er[i] = bk * fl;
                    qr[i] = qx[i] * fl;
                    const float gam = fl * fG[i];
                    qh[i] = qx[i] * gam;
                    en[i] = -(bk * gam);
                    kt[i] = km[i] * fTX[i];
                    kb[i] = kt[i] * fCG[i];
                }
                erf[s] = PR::make(er);
                qrf[s] = PR::make(qr);
                {
                    const Frag kmf = PR::make(km);
                    PR::mma(accA, PR::make(em), kmf);
                    PR::mma(accP, PR::make(qm), kmf);
                }
                PR::store8(&Qh[r * DKP + c0], qh);
                PR::store8(&En[r * DKP + c0], en);
                if (I < 3) PR::store8(&Kt[r * DKP + c0], kt);
                if (I < 2) {
                    float c8[8], ks[8];
                    if (I == 0) {
                        lds_read8f(tab + 17 * DK + c0, c8);
#pragma unroll
                        for (int i = 0; i < 8; ++i) ks[i] = kt[i] * c8[i];
                        PR::store8(&Ks[(0 * 16 + l16) * DKP + c0], ks);
                        lds_read8f(tab + 18 * DK + c0, c8);
#pragma unroll
                        for (int i = 0; i < 8; ++i) ks[i] = kt[i] * c8[i];
                        PR::store8(&Ks[(1 * 16 + l16) * DKP + c0], ks);
                    } else {
                        lds_read8f(tab + 19 * DK + c0, c8);
#pragma unroll
                        for (int i = 0; i < 8; ++i) ks[i] = kt[i] * c8[i];
                        PR::store8(&Ks[(2 * 16 + l16) * DKP + c0], ks);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) KbT[(c0 + i) * CHP + r] = (E)kb[i];
            }
            bool finite = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) finite = finite && __builtin_isfinite(accA[j]) && __builtin_isfinite(accP[j]);
            if (F16 && !__all(finite)) {
                // Strong decay inside the block: redo the diagonal Gram block with bf16 hi/lo
                // operands. The chunk row is reloaded (the registers already hold the next use).
                accA = f4{0.f, 0.f, 0.f, 0.f};
                accP = f4{0.f, 0.f, 0.f, 0.f};
                const int t = t0 + r;
                const bool valid = t < T;
                const long tok = ((long)bb * T + (valid ? t : 0)) * H + hh;
                float lg2v[CPL];
                if constexpr (AS) {
                    float x1 = lg2(valid ? load_one<BF16>(alpha, tok) : 1.f);
                    x1 += row_shr<1>(x1);
                    x1 += row_shr<2>(x1);
                    x1 += row_shr<4>(x1);
                    x1 += row_shr<8>(x1);
#pragma unroll
                    for (int e = 0; e < CPL; ++e) lg2v[e] = x1;
                } else {
#pragma unroll
                    for (int s = 0; s < NKS; ++s)
                        unpack8<BF16>(valid ? gload8<BF16>(alpha, tok * DK + 32 * s + 8 * g) : fill8<BF16>(1.f),
                                      &lg2v[8 * s]);
#pragma unroll
                    for (int e = 0; e < CPL; ++e) {
                        float x1 = lg2(lg2v[e]);
                        x1 += row_shr<1>(x1);
                        x1 += row_shr<2>(x1);
                        x1 += row_shr<4>(x1);
                        x1 += row_shr<8>(x1);
                        lg2v[e] = x1;
                    }
                }
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const int c0 = 32 * s + 8 * g;
                    float qx[8], kx[8], bx[8], X8[8], em[8], qm[8], km[8];
                    unpack8<BF16>(valid ? gload8<BF16>(q, tok * DK + c0) : fill8<BF16>(0.f), qx);
                    unpack8<BF16>(valid ? gload8<BF16>(k, tok * DK + c0) : fill8<BF16>(0.f), kx);
                    if constexpr (BS) {
                        const float be = valid ? load_one<BF16>(b, tok) : 0.f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) bx[i] = be;
                    } else {
                        unpack8<BF16>(valid ? gload8<BF16>(b, tok * DK + c0) : fill8<BF16>(0.f), bx);
                    }
                    lds_read8f(ldsX + I * DK + c0, X8);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float d = lg2v[8 * s + i] - X8[i];
                        const float fm = ex2(d);
                        em[i] = bx[i] * kx[i] * fm;
                        qm[i] = qx[i] * fm;
                        km[i] = kx[i] * ex2(-d);
                    }
                    PR::mma_wide(accA, em, km);
                    PR::mma_wide(accP, qm, km);
                }
            }
            // accumulator layout: row 4g+j of the block, column l16
            float4 at;
            at.x = (4 * g + 0) > l16 ? accA[0] : 0.f;
            at.y = (4 * g + 1) > l16 ? accA[1] : 0.f;
            at.z = (4 * g + 2) > l16 ? accA[2] : 0.f;
            at.w = (4 * g + 3) > l16 ? accA[3] : 0.f;
            *reinterpret_cast<float4*>(AdT + I * 256 + l16 * 16 + 4 * g) = at;  // A_II^T[col][row]
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 4 * g + j;
                Pm[(16 * I + rr) * CHP + 16 * I + l16] = (E)(rr >= l16 ? accP[j] : 0.f);
            }
            // U = w v for this lane's row and NCV value columns
            {
                float* up = U32 + r * UP + g * NCV;
#pragma unroll
                for (int u = 0; u < NCV / 8; ++u) {
                    float vx[8], wx[8];
                    unpack8<BF16>(keep_or<BF16>(rv[u], vrow, 0.f), vx);
                    if constexpr (BS) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) wx[i] = vrow ? rbs : 0.f;
                    } else {
                        unpack8<BF16>(keep_or<BF16>(rw[u], vrow, 0.f), wx);
                    }
                    float4* p = reinterpret_cast<float4*>(up + 8 * u);
                    p[0] = make_float4(wx[0] * vx[0], wx[1] * vx[1], wx[2] * vx[2], wx[3] * vx[3]);
                    p[1] = make_float4(wx[4] * vx[4], wx[5] * vx[5], wx[6] * vx[6], wx[7] * vx[7]);
                }
            }
        }
        lds_barrier();

        // ---------------- C: next chunk's loads; Gram blocks below the diagonal; T_II ----------------
        if (more) fetch(n + 1, 1);
        for (int J = 0; J < I; ++J) {
            const E* kb_ = (J == I - 1) ? Kt + (16 * J) * DKP
                                        : Ks + (16 * (I == 2 ? 0 : (J == 0 ? 1 : 2))) * DKP;
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const Frag kf = PR::lds8(kb_ + l16 * DKP + 32 * s + 8 * g);
                PR::mma(accA, erf[s], kf);
                PR::mma(accP, qrf[s], kf);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 16 * I + 4 * g + j;
                A32[rr * A32P + 16 * J + l16] = accA[j];
                Pm[rr * CHP + 16 * J + l16] = (E)accP[j];
            }
        }
        // T_II = (I + A_II)^-1, right-looking: once column m of T is final, it updates the rows
        // below. Column m + 1 of A_II is read from LDS while column m is applied.
        if (g == 0) {
            float acc[16], tc[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) acc[m] = 0.f;
            const float4* Ab4 = reinterpret_cast<const float4*>(AdT + I * 256);
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
            for (int m = 0; m < 16; ++m) Tm[(16 * I + m) * CHP + 16 * I + l16] = (E)tc[m];
        }
        lds_barrier();

        // ---------------- D: T10 = -T11 A10 T00 and T32 = -T33 A32 T22 ----------------
        if (wv == 1 || wv == 3) {
            const int Ib = wv, Jb = wv - 1;
            float af[8], bf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = A32[(16 * Ib + l16) * A32P + 16 * Jb + 4 * g + i];
                bf[i] = (float)Tm[(16 * Jb + 4 * g + i) * CHP + 16 * Jb + l16];
                af[i + 4] = bf[i + 4] = 0.f;
            }
            f4 X = {0.f, 0.f, 0.f, 0.f};
            PR::mma(X, PR::make(af), PR::make(bf));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = (float)Tm[(16 * Ib + l16) * CHP + 16 * Ib + 4 * g + i];
                bf[i] = X[i];
            }
            f4 Y = {0.f, 0.f, 0.f, 0.f};
            PR::mma(Y, PR::make(af), PR::make(bf));
#pragma unroll
            for (int j = 0; j < 4; ++j) Tm[(16 * Ib + 4 * g + j) * CHP + 16 * Jb + l16] = (E)(-Y[j]);
        }
        lds_barrier();

        // ---------------- E: T[32:, :32] = -T[32:, 32:] A[32:, :32] T[:32, :32] ----------------
        if (wv < 2) {
            const int Jb = wv;
            f4 Yt[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int Ib = 2 + u;
                float af[8], bf[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    af[i] = A32[(16 * Ib + l16) * A32P + kap(g, i)];
                    bf[i] = (float)Tm[kap(g, i) * CHP + 16 * Jb + l16];
                }
                Yt[u] = f4{0.f, 0.f, 0.f, 0.f};
                PR::mma(Yt[u], PR::make(af), PR::make(bf));
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
                const E* row = &Tm[(16 * Ib + l16) * CHP + 32];
                const Frag tf = PR::lds_pair(row + 4 * g, row + 16 + 4 * g);
                f4 Z = {0.f, 0.f, 0.f, 0.f};
                PR::mma(Z, tf, yf);
#pragma unroll
                for (int j = 0; j < 4; ++j) Tm[(16 * Ib + 4 * g + j) * CHP + 16 * Jb + l16] = (E)(-Z[j]);
            }
        }
        lds_barrier();

        // ---------------- F: the state chain for this wave's 16 columns ----------------
        if (more) fetch(n + 1, 2);
        if (chain) {
            // D' starts as U = w v (times sc for fp16 operands, see chunk_common.h rescale_state)
            f4 D[4], O[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int j = 0; j < 4; ++j) D[mt][j] = U32[(16 * mt + 4 * g + j) * UP + 16 * wv + l16];
            if constexpr (F16) rescale_state<NMK>(Sacc, D, esc, sc, isc);
            // state as B operand: K-step s covers channels 32s..32s+31 = tiles 2s, 2s+1
            Frag Sf[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                float sv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sv[i] = Sacc[2 * s][i];
                    sv[i + 4] = Sacc[2 * s + 1][i];
                }
                Sf[s] = PR::make(sv);
            }
            // D' = U - E_hat S, and O^T = S^T Q_hat^T: the state fragments serve as the A
            // operand of the transposed product, so O^T tile nt holds, per lane, four
            // consecutive state columns (rows 4g..4g+3) of token 16 nt + l16.
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                O[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const E* er_ = &En[(16 * mt + l16) * DKP + 32 * s];
                    const E* qr_ = &Qh[(16 * mt + l16) * DKP + 32 * s];
                    PR::mma(D[mt], PR::lds_pair(er_ + 4 * g, er_ + 16 + 4 * g), Sf[s]);
                    PR::mma(O[mt], Sf[s], PR::lds_pair(qr_ + 4 * g, qr_ + 16 + 4 * g));
                }
            }
            if (more) fetch(n + 1, 3);
            // Delta = T D' (T lower triangular: token K-steps s2 <= mt / 2)
            Frag Df[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float dv_[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dv_[i] = D[2 * s2][i];
                    dv_[i + 4] = D[2 * s2 + 1][i];
                }
                Df[s2] = PR::make(dv_);
            }
            f4 Dl[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                Dl[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 <= mt / 2; ++s2) {
                    const E* tr = &Tm[(16 * mt + l16) * CHP + 32 * s2];
                    PR::mma(Dl[mt], PR::lds_pair(tr + 4 * g, tr + 16 + 4 * g), Df[s2]);
                }
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float dv_[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dv_[i] = Dl[2 * s2][i];
                    dv_[i + 4] = Dl[2 * s2 + 1][i];
                }
                Df[s2] = PR::make(dv_);
            }
            // O^T += Delta^T P^T (P lower triangular), then store four columns per lane
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                for (int s2 = 0; s2 <= nt / 2; ++s2) {
                    const E* pr = &Pm[(16 * nt + l16) * CHP + 32 * s2];
                    PR::mma(O[nt], Df[s2], PR::lds_pair(pr + 4 * g, pr + 16 + 4 * g));
                }
                const __amdgpu_buffer_rsrc_t rs_o = rows_rsrc(o, (long)bb * T, t0, T, (unsigned)(H * DV * 4), CH);
                const unsigned row = (unsigned)(16 * nt + l16);
                store4(rs_o, ((row * H + hh) * DV + tile * DVT + 16 * wv + 4 * g) * 4u, O[nt][0] * isc, O[nt][1] * isc,
                       O[nt][2] * isc, O[nt][3] * isc);
            }
            // S <- Diag(gamma_last) S + K_bar^T Delta
#pragma unroll
            for (int mk = 0; mk < NMK; ++mk) {
                const float4 gc = *reinterpret_cast<const float4*>(tab + 16 * DK + 16 * mk + 4 * g);
                Sacc[mk][0] *= gc.x;
                Sacc[mk][1] *= gc.y;
                Sacc[mk][2] *= gc.z;
                Sacc[mk][3] *= gc.w;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const E* kr = &KbT[(16 * mk + l16) * CHP + 32 * s2];
                    PR::mma(Sacc[mk], PR::lds_pair(kr + 4 * g, kr + 16 + 4 * g), Df[s2]);
                }
            }
        } else if (more) {
            fetch(n + 1, 3);
        }
        lds_barrier();
    }

    if (chain && S_out) {
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S_out[sbase + (long)(16 * mk + 4 * g + j) * DV + mycol] = Sacc[mk][j] * isc;
    }
}

template <int DK, bool BF16, bool AS, bool BS>
hipError_t launch_t(const ChunkArgs& a, hipStream_t s) {
    constexpr int DVT = DK < 64 ? DK : 64;
    const int tiles = a.DV / DVT;
    const int bh = a.B * a.H;
    const int groups = (bh + 7) / 8;
    const int blocks = groups * 8 * tiles;
    hipLaunchKernelGGL((chunk_kernel<DK, DVT, BF16, AS, BS>), dim3(blocks), dim3(256), 0, s, a.q,
                       a.k, a.v, a.alpha, a.b, a.w, a.S0, a.o, a.S_out, a.B, a.T, a.H, a.DV);
    return hipGetLastError();
}

template <int DK, bool BF16>
hipError_t launch_flags(const ChunkArgs& a, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_t<DK, BF16, false, false>(a, s);
        case 1: return launch_t<DK, BF16, true, false>(a, s);
        case 2: return launch_t<DK, BF16, false, true>(a, s);
        default: return launch_t<DK, BF16, true, true>(a, s);
    }
}

}  // namespace

bool chunk_supported(int T, int H, int DK, int DV, bool bf16) {
    if (DK != DV || T < 0) return false;
    if (bf16) return DK == 32 || DK == 64 || DK == 128;
    return DK == 32 || DK == 64;  // fp32 operand tiles of d = 128 exceed the LDS budget
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t s) {
    if (!chunk_supported(a.T, a.H, a.DK, a.DV, a.bf16)) return hipErrorNotSupported;
    if (a.bf16) {
        switch (a.DK) {
            case 32: return launch_flags<32, true>(a, s);
            case 64: return launch_flags<64, true>(a, s);
            default: return launch_flags<128, true>(a, s);
        }
    }
    return a.DK == 32 ? launch_flags<32, false>(a, s) : launch_flags<64, false>(a, s);
}

}  // namespace gdn2
