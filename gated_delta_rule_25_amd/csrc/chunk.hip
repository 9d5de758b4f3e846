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
// columns of S evolve independently given W and U~, so tiles need no communication. The
// sequence is walked chunk by chunk:
//   A  wave I loads token rows 16I..16I+15 (lane = row, 8 channels per K-step) and scans the
//      log2-decay over its 16 rows with lane shuffles; block totals go through LDS.
//   B  factors: Q_hat, E_hat^T, K_bar^T, U^T and the block-referenced K~ go to LDS; the
//      diagonal 16x16 Gram blocks are formed in registers. Their factors are referenced to
//      the block's 8th row, so no factor exceeds the decay of 8 tokens, and they use a bf16
//      hi/lo split (three passes) with the fp32 exponent range.
//   C  Gram blocks below the diagonal: row side exp2(local), column side
//      exp2(blocktot - local), both <= 1, times exp2(G_I - G_{J+1}) <= 1 for non-adjacent
//      blocks; one fp16 pass. Then each wave inverts its 16x16 diagonal block of (I + A) by
//      fp32 forward substitution.
//   D,E  the 16x16 inverses are merged into the 64x64 T at 32 and 64 rows:
//      T21 = -T22 A21 T11 per 32-row half, then T[32:,:32] = -T[32:,32:] A[32:,:32] T[:32,:32].
//   F  W = T E_hat (stored negated), then the state chain: each wave owns 16 state columns,
//      held in accumulator registers (fp32) for the whole sequence, and computes
//      Delta = U~ + (-W) S, O = Q_hat S + P Delta, S = gamma_last S + K_bar^T Delta.
//      Accumulator tiles feed the next product directly: operand k-slots are chosen to match
//      the accumulator layout (kap below), and the A operands read LDS in the same order.
//
// Precision: with bf16 inputs the products take fp16 operands (fp32 accumulation, fp32 state,
// fp32 o); with fp32 inputs they take fp32 operands (v_mfma_f32_16x16x4_f32).
#include "common.h"
#include "kernels.h"

namespace gdn2 {

namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length

// k-slot i of lane group g inside a 32-wide K-step, matching two stacked accumulator tiles:
// slots 0..3 are rows 4g..4g+3 of the first tile, slots 4..7 rows 4g..4g+3 of the second.
__device__ __forceinline__ int kap(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// ---- operand precision policies ---------------------------------------------------------
template <bool F16>
struct Prec;

template <>
struct Prec<true> {
    using E = _Float16;
    static constexpr int kPad = 8;  // 16 bytes of row padding
    using Frag = h8;
    __device__ static Frag make(const float* x) {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (_Float16)x[i];
        return f;
    }
    // slots 0..3 from p0[0..3], slots 4..7 from p1[0..3]
    __device__ static Frag lds_pair(const E* p0, const E* p1) {
        const h4 a = *reinterpret_cast<const h4*>(p0);
        const h4 b = *reinterpret_cast<const h4*>(p1);
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ static Frag lds8(const E* p) { return *reinterpret_cast<const h8*>(p); }
    __device__ static void store8(E* p, const float* x) { *reinterpret_cast<h8*>(p) = make(x); }
    __device__ static void mma(f4& c, const Frag& a, const Frag& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    // Gram diagonal blocks: bf16 hi/lo split of both operands, hi*hi + hi*lo + lo*hi.
    __device__ static void mma_wide(f4& c, const float* a, const float* b) {
        b8 ah, al, bh, bl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const __bf16 x = (__bf16)a[i];
            ah[i] = x;
            al[i] = (__bf16)(a[i] - (float)x);
            const __bf16 y = (__bf16)b[i];
            bh[i] = y;
            bl[i] = (__bf16)(b[i] - (float)y);
        }
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
    }
};

template <>
struct Prec<false> {
    using E = float;
    static constexpr int kPad = 4;
    struct Frag {
        float v[8];
    };
    __device__ static Frag make(const float* x) {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = x[i];
        return f;
    }
    __device__ static Frag lds_pair(const E* p0, const E* p1) {
        const float4 a = *reinterpret_cast<const float4*>(p0);
        const float4 b = *reinterpret_cast<const float4*>(p1);
        return Frag{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
    }
    __device__ static Frag lds8(const E* p) { return lds_pair(p, p + 4); }
    __device__ static void store8(E* p, const float* x) {
        reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    // 16x16x4 fp32 passes: pass i contracts slot i of every lane group.
    __device__ static void mma(f4& c, const Frag& a, const Frag& b) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
    }
    __device__ static void mma_wide(f4& c, const float* a, const float* b) {
        mma(c, make(a), make(b));
    }
};

// ---- LDS layout ----------------------------------------------------------------------------
template <int DK, int DVT, bool F16>
struct Smem {
    using E = typename Prec<F16>::E;
    static constexpr int PAD = Prec<F16>::kPad;
    static constexpr int DKP = DK + PAD;   // token-major rows (channels)
    static constexpr int CHP = CH + PAD;   // channel- or token-major rows of 64 tokens
    static constexpr int A32P = CH + 4;    // fp32 A rows
    // byte offsets
    static constexpr int oTot = 0;                                  // float [4][DK]
    static constexpr int oGC = oTot + 4 * DK * 4;                   // float [DK]
    static constexpr int oQh = oGC + DK * 4;                        // E [64][DKP]
    static constexpr int oEhT = oQh + CH * DKP * (int)sizeof(E);    // E [DK][CHP]
    static constexpr int oKbT = oEhT + DK * CHP * (int)sizeof(E);   // E [DK][CHP]
    static constexpr int oUT = oKbT + DK * CHP * (int)sizeof(E);    // E [DVT][CHP]
    static constexpr int oP = oUT + DVT * CHP * (int)sizeof(E);     // E [64][CHP]
    static constexpr int oTm = oP + CH * CHP * (int)sizeof(E);      // E [64][CHP]
    static constexpr int oR = oTm + CH * CHP * (int)sizeof(E);      // union region
    static constexpr int oKt = oR;                                  // E [48][DKP]
    static constexpr int oA = oKt + 48 * DKP * (int)sizeof(E);      // float [64][A32P]
    static constexpr int oWn = oR;                                  // E [64][DKP] (after A dies)
    static constexpr int endR1 = oA + CH * A32P * 4;
    static constexpr int endR2 = oWn + CH * DKP * (int)sizeof(E);
    static constexpr int bytes = endR1 > endR2 ? endR1 : endR2;
    static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
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
    constexpr int NKS = DK / 32;   // K-steps over channels
    constexpr int NMK = DK / 16;   // 16-row tiles over channels
    constexpr int NWC = DVT / 16;  // waves owning state columns
    constexpr int CPL = DK / 4;    // channels per lane in the token-major layout
    constexpr int DKP = SM::DKP, CHP = SM::CHP, A32P = SM::A32P;

    __shared__ __attribute__((aligned(16))) char smem[SM::bytes];
    float* ldsTot = reinterpret_cast<float*>(smem + SM::oTot);
    float* ldsGC = reinterpret_cast<float*>(smem + SM::oGC);
    E* Qh = reinterpret_cast<E*>(smem + SM::oQh);
    E* EhT = reinterpret_cast<E*>(smem + SM::oEhT);
    E* KbT = reinterpret_cast<E*>(smem + SM::oKbT);
    E* UT = reinterpret_cast<E*>(smem + SM::oUT);
    E* Pm = reinterpret_cast<E*>(smem + SM::oP);
    E* Tm = reinterpret_cast<E*>(smem + SM::oTm);
    E* Kt = reinterpret_cast<E*>(smem + SM::oKt);
    float* A32 = reinterpret_cast<float*>(smem + SM::oA);
    E* Wn = reinterpret_cast<E*>(smem + SM::oWn);

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

    const int nch = (T + CH - 1) / CH;
    for (int n = 0; n < nch; ++n) {
        const int t0 = n * CH;
        const int L = min(CH, T - t0);

        // ---------------- A: loads and in-block log2-decay scan ----------------
        const int I = wv;
        const int r = 16 * I + l16;
        const bool valid = r < L;
        const long tok = ((long)bb * T + (t0 + (valid ? r : 0))) * H + hh;
        float qv[CPL], kv[CPL], bv[CPL], lg[CPL];  // index 8s+i <-> channel 32s + 8g + i
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int c0 = 32 * s + 8 * g;
            if (valid) {
                load_vec<8, BF16>(q, tok * DK + c0, &qv[8 * s]);
                load_vec<8, BF16>(k, tok * DK + c0, &kv[8 * s]);
                if constexpr (!BS) load_vec<8, BF16>(b, tok * DK + c0, &bv[8 * s]);
                if constexpr (!AS) load_vec<8, BF16>(alpha, tok * DK + c0, &lg[8 * s]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    qv[8 * s + i] = kv[8 * s + i] = bv[8 * s + i] = 0.f;
                    lg[8 * s + i] = 1.f;
                }
            }
        }
        if constexpr (AS) {
            const float a = valid ? load_one<BF16>(alpha, tok) : 1.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) lg[e] = a;
        }
        if constexpr (BS) {
            const float be = valid ? load_one<BF16>(b, tok) : 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) bv[e] = be;
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) lg[e] = lg2(lg[e]);
        // inclusive scan over the 16 rows of the block (lanes l16 = 0..15 of each group)
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const float y = __shfl_up(lg[e], d, 16);
                if (l16 >= d) lg[e] += y;
            }
        }
        if (l16 == 15) {
#pragma unroll
            for (int s = 0; s < NKS; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i) ldsTot[I * DK + 32 * s + 8 * g + i] = lg[8 * s + i];
        }
        __syncthreads();

        // ---------------- B: factors, LDS operand tiles, diagonal Gram blocks ----------------
        float er[CPL], qr[CPL];  // row-side Gram factors referenced to the block start
        {
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                float qh[8], eh[8], kb[8], kt[8], em[8], qm[8], km[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = 8 * s + i;
                    const int c = 32 * s + 8 * g + i;
                    float Gi = 0.f, gC = 0.f;
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        const float t = ldsTot[J * DK + c];
                        if (J < I) Gi += t;
                        gC += t;
                    }
                    const float totI = ldsTot[I * DK + c];
                    const float X = __shfl(lg[e], 7, 16);  // local value at the block's 8th row
                    const float Gam = Gi + lg[e];
                    const float gam = ex2(Gam);
                    const float ebk = bv[e] * kv[e];
                    qh[i] = qv[e] * gam;
                    eh[i] = ebk * gam;
                    kb[i] = kv[e] * ex2(gC - Gam);
                    kt[i] = kv[e] * ex2(totI - lg[e]);
                    const float fl = ex2(lg[e]);
                    er[e] = ebk * fl;
                    qr[e] = qv[e] * fl;
                    const float fm = ex2(lg[e] - X);
                    em[i] = ebk * fm;
                    qm[i] = qv[e] * fm;
                    km[i] = kv[e] * ex2(X - lg[e]);
                    if (wv == 0 && l16 == 0) ldsGC[c] = ex2(gC);
                }
                const int c0 = 32 * s + 8 * g;
                PR::store8(&Qh[r * DKP + c0], qh);
                if (I < 3) PR::store8(&Kt[r * DKP + c0], kt);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    EhT[(c0 + i) * CHP + r] = (E)eh[i];
                    KbT[(c0 + i) * CHP + r] = (E)kb[i];
                }
                PR::mma_wide(accA, em, km);
                PR::mma_wide(accP, qm, km);
            }
            // accumulator layout: row 4g+j of the block, column l16
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 4 * g + j;
                A32[(16 * I + rr) * A32P + 16 * I + l16] = rr > l16 ? accA[j] : 0.f;
                Pm[(16 * I + rr) * CHP + 16 * I + l16] = (E)(rr >= l16 ? accP[j] : 0.f);
            }
            // U^T for this workgroup's value tile: lane (row r, group g) covers DVT/4 columns
            {
                constexpr int NC = DVT / 4;
                float vv[NC], ww[NC];
                const int cl0 = g * NC;
                const long vtok = ((long)bb * T + (t0 + (valid ? r : 0))) * H + hh;
                if (valid) {
                    load_vec<NC, BF16>(v, vtok * DV + tile * DVT + cl0, vv);
                    if constexpr (BS) {
#pragma unroll
                        for (int i = 0; i < NC; ++i) ww[i] = bv[0];
                    } else {
                        load_vec<NC, BF16>(w, vtok * DV + tile * DVT + cl0, ww);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < NC; ++i) vv[i] = ww[i] = 0.f;
                }
#pragma unroll
                for (int i = 0; i < NC; ++i) UT[(cl0 + i) * CHP + r] = (E)(ww[i] * vv[i]);
            }
        }
        __syncthreads();

        // ---------------- C: Gram blocks below the diagonal; diagonal UT inverses ----------------
        for (int J = 0; J < I; ++J) {
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                float ea[8], qa[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = 8 * s + i;
                    const int c = 32 * s + 8 * g + i;
                    float cij = 1.f;
                    if (J < I - 1) {  // exp2(G_I - G_{J+1}) = exp2(sum of the blocks between)
                        float between = 0.f;
                        for (int Jm = J + 1; Jm < I; ++Jm) between += ldsTot[Jm * DK + c];
                        cij = ex2(between);
                    }
                    ea[i] = er[e] * cij;
                    qa[i] = qr[e] * cij;
                }
                const Frag kf = PR::lds8(&Kt[(16 * J + l16) * DKP + 32 * s + 8 * g]);
                PR::mma(accA, PR::make(ea), kf);
                PR::mma(accP, PR::make(qa), kf);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 16 * I + 4 * g + j;
                A32[rr * A32P + 16 * J + l16] = accA[j];
                Pm[rr * CHP + 16 * J + l16] = (E)accP[j];
            }
        }
        // T_II = (I + A_II)^-1 by forward substitution; lane l16 of group 0 owns column l16
        if (g == 0) {
            float tc[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) tc[m] = (m == l16) ? 1.f : 0.f;
            const float* Ab = A32 + (16 * I) * A32P + 16 * I;
#pragma unroll
            for (int rr = 1; rr < 16; ++rr) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < rr; ++m) acc = fmaf(Ab[rr * A32P + m], tc[m], acc);
                if (rr > l16) tc[rr] = -acc;
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) Tm[(16 * I + m) * CHP + 16 * I + l16] = (E)tc[m];
        }
        __syncthreads();

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
        __syncthreads();

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
        __syncthreads();

        // ---------------- F1: -W = -T E_hat into LDS (overlays K~ and A) ----------------
        for (int nt = wv; nt < NMK; nt += 4) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= mt / 2; ++s) {
                    const E* tr = &Tm[(16 * mt + l16) * CHP + 32 * s];
                    const E* er_ = &EhT[(16 * nt + l16) * CHP + 32 * s];
                    PR::mma(acc, PR::lds_pair(tr + 4 * g, tr + 16 + 4 * g),
                            PR::lds_pair(er_ + 4 * g, er_ + 16 + 4 * g));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) Wn[(16 * mt + 4 * g + j) * DKP + 16 * nt + l16] = (E)(-acc[j]);
            }
        }
        __syncthreads();

        // ---------------- F2: the state chain for this wave's 16 columns ----------------
        if (chain) {
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
            f4 D[4], O[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                D[mt] = f4{0.f, 0.f, 0.f, 0.f};
                O[mt] = f4{0.f, 0.f, 0.f, 0.f};
                // U~ = T U
#pragma unroll
                for (int s = 0; s <= mt / 2; ++s) {
                    const E* tr = &Tm[(16 * mt + l16) * CHP + 32 * s];
                    const E* ur = &UT[(16 * wv + l16) * CHP + 32 * s];
                    PR::mma(D[mt], PR::lds_pair(tr + 4 * g, tr + 16 + 4 * g),
                            PR::lds_pair(ur + 4 * g, ur + 16 + 4 * g));
                }
                // Delta = U~ + (-W) S ; O = Q_hat S
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const E* wr = &Wn[(16 * mt + l16) * DKP + 32 * s];
                    const E* qr_ = &Qh[(16 * mt + l16) * DKP + 32 * s];
                    PR::mma(D[mt], PR::lds_pair(wr + 4 * g, wr + 16 + 4 * g), Sf[s]);
                    PR::mma(O[mt], PR::lds_pair(qr_ + 4 * g, qr_ + 16 + 4 * g), Sf[s]);
                }
            }
            // Delta as B operand over tokens: K-step s2 covers tokens 32 s2 .. 32 s2 + 31
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
            // O += P Delta, then store the valid rows
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int s2 = 0; s2 <= mt / 2; ++s2) {
                    const E* pr = &Pm[(16 * mt + l16) * CHP + 32 * s2];
                    PR::mma(O[mt], PR::lds_pair(pr + 4 * g, pr + 16 + 4 * g), Df[s2]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * mt + 4 * g + j;
                    if (row < L) o[(((long)bb * T + t0 + row) * H + hh) * DV + mycol] = O[mt][j];
                }
            }
            // S <- Diag(gamma_last) S + K_bar^T Delta
#pragma unroll
            for (int mk = 0; mk < NMK; ++mk) {
#pragma unroll
                for (int j = 0; j < 4; ++j) Sacc[mk][j] *= ldsGC[16 * mk + 4 * g + j];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const E* kr = &KbT[(16 * mk + l16) * CHP + 32 * s2];
                    PR::mma(Sacc[mk], PR::lds_pair(kr + 4 * g, kr + 16 + 4 * g), Df[s2]);
                }
            }
        }
        __syncthreads();
    }

    if (chain && S_out) {
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S_out[sbase + (long)(16 * mk + 4 * g + j) * DV + mycol] = Sacc[mk][j];
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

bool chunk_supported(int DK, int DV, bool bf16) {
    if (DK != DV) return false;
    if (bf16) return DK == 32 || DK == 64 || DK == 128;
    return DK == 32 || DK == 64;
}

size_t chunk_workspace_bytes(int B, int T, int H, int DK, int DV, bool bf16, uint32_t flags) {
    return 0;
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t s) {
    if (!chunk_supported(a.DK, a.DV, a.bf16)) return hipErrorNotSupported;
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
