// chunk_fused.hip -- chunkwise (C = 64) Gated DeltaNet-2 prefill in one kernel on gfx950, with the
// state-free work of the next chunk overlapped with the state chain of the current one.
//
// Same method and arithmetic as the two-kernel path [page "NVIDIA представила Gated DeltaNet-2 с
// канал-wise гейтами …", paragraph "Реализация": chunkwise WY form, C = 64, the cumulative
// channel-wise decay absorbed into the rank-1 factors], for bf16 inputs (fp16 matrix-core
// operands, fp32 accumulation and state). The difference is where the per-chunk operands live:
// the two-kernel path writes every chunk's operand block (Q_hat, -E_hat, K_bar^T, P, T,
// gamma_last) to HBM and reads it back; here the block never leaves the CU.
//
// One workgroup of 8 wavefronts per (b, h, tile of 64 value columns):
//   waves 0..3  chain: each owns 16 state columns, held in fp32 accumulators for the whole
//               sequence, and runs chunk n from LDS buffer n % 2:
//                 D' = U - E_hat S,  Delta = T D',  O^T = S^T Q_hat^T + Delta^T P^T,
//                 S <- Diag(gamma_last) S + K_bar^T Delta
//               (v, w of the next chunk copied into a private LDS slot, o stored per chunk).
//   waves 4..7  prep: build chunk n + 1's block in buffer (n + 1) % 2 -- decay scan, factors,
//               Gram blocks, the UT inverse T -- with the next chunk's q, k, alpha, b rows already
//               in registers (their loads are issued one chunk ahead).
// One workgroup barrier per chunk hands the buffers over. The prep waves' own phases are ordered
// by a counter in LDS that only they wait on, so the chain waves never stop at those steps.
//
// LDS (d = 128): two blocks of 62,208 B and the prep scratch: scan totals, decay tables, diagonal
// A blocks, the key rows of the Gram blocks and the A rows of the inverse's merges (38.9 KB), with
// 16-byte (key rows) and 8-byte (A rows) units XOR-permuted by row so that the 16 rows a fragment
// read touches fall in distinct banks without padding: 163,408 of the 163,840 bytes. The chain
// waves load their v, w columns straight into registers, one chunk ahead.
//
// HBM traffic per head-token is the algorithmic one: q, k, alpha, b, v, w read, o written (the two
// value tiles of a head run on one XCD, so its q, k, alpha, b are fetched once into that L2).
#include "chunk_blob.h"
#include "kernels.h"

namespace gdn2 {

namespace {

using namespace chunk;

constexpr int kFusedThreads = 512;  // 4 chain + 4 prep wavefronts

template <int DK>
struct FusedSmem {
    using BL = Blob<DK, true>;
    static constexpr int DVT = DK < 64 ? DK : 64;          // value columns per workgroup
    static constexpr int NWC = DVT / 16;                   // chain waves
    static constexpr int ADS = 260;                        // diagonal A^T block stride (floats)
    static constexpr int oBuf0 = 0;
    static constexpr int oBuf1 = BL::bytes;
    // decay tables per (block I, channel), exp2 of: 0..3 tot_I, 4..7 G_I, 8..11 gC - G_{I+1},
    // 12 gC, 13 tot_1, 14 tot_1 + tot_2, 15 tot_2 (tot_I: block I's total log2-decay, G_I: the
    // earlier blocks' total, gC: the chunk's)
    static constexpr int kTab = 16;
    static constexpr int oTot = 2 * BL::bytes;             // float [4][DK]
    static constexpr int oTab = oTot + 4 * DK * 4;         // float [kTab][DK]
    static constexpr int oAd = oTab + kTab * DK * 4;       // float [4][ADS]
    static constexpr int oKt = oAd + 4 * ADS * 4;          // fp16 [48][DK], 16-byte units swizzled
    static constexpr int oA = oKt + 48 * DK * 2;           // fp16 [64][64], 8-byte units swizzled
    static constexpr int oCtr = oA + CH * CH * 2;          // unsigned: prep-wave barrier counter
    static constexpr int bytes = oCtr + 16;
    static_assert(BL::bytes % 256 == 0 && oTot % 16 == 0 && oKt % 16 == 0, "alignment");
    static_assert(bytes <= 160 * 1024, "LDS budget");
    // key row r, channel c (c a multiple of 8 for 16-byte accesses): unit c / 8 XOR (r mod 16)
    __device__ static int kt(int r, int c) { return r * DK + ((((c >> 3) ^ (r & 15)) & (DK / 8 - 1)) << 3) + (c & 7); }
    // A row r, column c: 4-element unit c / 4 XOR (r mod 16)
    __device__ static int ar(int r, int c) { return r * CH + ((((c >> 2) ^ (r & 15)) & 15) << 2) + (c & 3); }
};

// Barrier over the four prep waves: each adds one to an LDS counter and waits until all four
// have arrived at this step (target advances by 4 per step). The wait polls the counter without
// sleeping between reads (a sleep of one unit, 64 cycles, between polls measured 1.3% slower on
// the whole call) and is bounded at 2^22 polls (well under a second), so a wave can never hang
// here.
__device__ __forceinline__ void prep_sync(unsigned* ctr, unsigned& target, int lane) {
    target += 4u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (unsigned spin = 0; spin < (1u << 22); ++spin) {
        if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Issue-order hint for a run of P products that each read one LDS operand fragment.
template <int P, int LA = 4, int MPR = 1>
__device__ __forceinline__ void fused_lookahead() {
    constexpr int la = P < LA ? P : LA;
    __builtin_amdgcn_sched_group_barrier(0x100, la, 0);
#pragma unroll
    for (int i = 0; i < P - la; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, la * MPR, 0);
}

// Eight elements c0..c0+7 of row r of -E_hat or Q_hat into a block in LDS (two 8-byte units).
template <typename BL>
__device__ __forceinline__ void put8_units(_Float16* base, int r, int c0, const float* x) {
    h4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = (_Float16)x[i];
        b[i] = (_Float16)x[i + 4];
    }
    *reinterpret_cast<h4*>(base + BL::en(r, c0)) = a;
    *reinterpret_cast<h4*>(base + BL::en(r, c0 + 4)) = b;
}

// The diagonal 16x16 Gram blocks of one 16-row block, A and P, recomputed with bf16 hi/lo operands
// (three passes, fp32 exponent range) when the one-pass fp16 products overflowed: the lane's row
// (token index tok) is read again, its log2-decay scanned again over the block's 16 rows, and the
// factors referenced to the block's 8th row, so that no factor exceeds the decay across 8 rows.
struct DiagPair {
    f4 a, p;
};

template <int DK, bool AS, bool BS, int PRO>
__device__ __noinline__ DiagPair diag_gram_wide(const void* q, const void* k, const void* alpha, const void* b, long tok,
                                                bool valid, float nq, float nk, int lane) {
    const int g = lane >> 4, ref = (lane & 48) | 7;  // the block's 8th row holds the reference
    constexpr bool BF16 = true, L2N = (PRO & 1) != 0, GL = (PRO & 2) != 0;
    constexpr int NKS = DK / 32, CPL = DK / 4;
    using PR = Prec<true>;
    float lgv[CPL];
    if constexpr (AS) {
        const float a1 = load_one<BF16>(alpha, tok);
        float x1 = GL ? (valid ? lg2_sigmoid(a1) : 0.f) : lg2(valid ? a1 : 1.f);
        x1 += row_shr<1>(x1);
        x1 += row_shr<2>(x1);
        x1 += row_shr<4>(x1);
        x1 += row_shr<8>(x1);
#pragma unroll
        for (int e = 0; e < CPL; ++e) lgv[e] = x1;
    } else {
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            unpack8<BF16>(keep_or<BF16>(gload8<BF16>(alpha, tok * DK + 32 * s + 8 * g), valid, GL ? INFINITY : 1.f),
                          &lgv[8 * s]);
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            float x1 = GL ? lg2_sigmoid(lgv[e]) : lg2(lgv[e]);
            x1 += row_shr<1>(x1);
            x1 += row_shr<2>(x1);
            x1 += row_shr<4>(x1);
            x1 += row_shr<8>(x1);
            lgv[e] = x1;
        }
    }
    const float bsc = BS ? load_one<BF16>(b, tok) : 0.f;
    DiagPair r{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const int c0 = 32 * s + 8 * g;
        float qx[8], kx[8], bx[8], X8[8], em[8], qm[8], km[8];
        unpack8<BF16>(keep_or<BF16>(gload8<BF16>(q, tok * DK + c0), valid, 0.f), qx);
        unpack8<BF16>(keep_or<BF16>(gload8<BF16>(k, tok * DK + c0), valid, 0.f), kx);
        if constexpr (BS) {
            const float be = GL ? sigmoidf_(bsc) : bsc;
#pragma unroll
            for (int i = 0; i < 8; ++i) bx[i] = valid ? be : 0.f;
        } else {
            unpack8<BF16>(keep_or<BF16>(gload8<BF16>(b, tok * DK + c0), valid, GL ? -INFINITY : 0.f), bx);
            if constexpr (GL) {
#pragma unroll
                for (int i = 0; i < 8; ++i) bx[i] = sigmoidf_(bx[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) X8[i] = __shfl(lgv[8 * s + i], ref);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (L2N) {
                qx[i] *= nq;
                kx[i] *= nk;
            }
            const float d = lgv[8 * s + i] - X8[i];
            const float fm = ex2(d);
            em[i] = bx[i] * kx[i] * fm;
            qm[i] = qx[i] * fm;
            km[i] = kx[i] * ex2(-d);
        }
        PR::mma_wide(r.a, em, km);
        PR::mma_wide(r.p, qm, km);
    }
    return r;
}

// PRO (prologue): bit 0, q and k are L2-normalised per token here; bit 1, alpha, b, w (or beta)
// arrive as pre-activations.
template <int DK, bool AS, bool BS, int PRO>
__global__ void __launch_bounds__(kFusedThreads, 1)
fused_kernel(const void* q, const void* k, const void* v, const void* alpha, const void* b, const void* w,
             const float* S0, float* o, float* S_out, int B, int T, int H, int DV) {
    constexpr bool BF16 = true;
    using PR = Prec<true>;
    using E = _Float16;
    using Frag = PR::Frag;
    using BL = Blob<DK, true>;
    using SM = FusedSmem<DK>;
    constexpr int NKS = DK / 32, NMK = DK / 16, CPL = DK / 4;
    constexpr int DVT = SM::DVT, NWC = SM::NWC;
    constexpr bool L2N = (PRO & 1) != 0, GL = (PRO & 2) != 0;

    __shared__ __attribute__((aligned(16))) char smem[SM::oTot];              // the two blocks
    __shared__ __attribute__((aligned(16))) char sps[SM::bytes - SM::oTot];  // prep scratch
    float* ldsTot = reinterpret_cast<float*>(sps);
    float* tab = reinterpret_cast<float*>(sps + (SM::oTab - SM::oTot));
    float* AdT = reinterpret_cast<float*>(sps + (SM::oAd - SM::oTot));
    unsigned* ctr = reinterpret_cast<unsigned*>(sps + (SM::oCtr - SM::oTot));

    // (the wave index through readfirstlane: a scalar, so the role branches below are uniform and
    // each role's barriers are reached by whole wavefronts)
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    // Work item, as in the chain kernel: workgroups are dealt round-robin over the 8 XCDs, and the
    // value tiles of one (b, h) sit 8 apart, on one XCD, sharing q, k, alpha, b in its L2.
    const int tiles = DV / DVT;
    const int BH = B * H;
    const int grp = blockIdx.x / (8 * tiles), within = blockIdx.x % (8 * tiles);
    const int tile = within / 8;
    const int bh = grp * 8 + (within % 8);
    if (bh >= BH) return;  // uniform over the workgroup
    const int hh = bh % H;
    const long tbase = (long)(bh / H) * T;  // first token row of this sequence
    const int nch = (T + CH - 1) / CH;
    const bool chain = wv < NWC;
    const bool prep = wv >= 4;

    if (threadIdx.x == 0) *ctr = 0u;
    // upper blocks of T and P that the block layout stores are zero; nothing writes them later
    for (int idx = threadIdx.x; idx < 2 * CH * CH; idx += kFusedThreads) {
        const int which = idx / (CH * CH), rr = (idx / CH) % CH, cc = idx % CH;
        if ((cc >> 4) > (rr >> 4) && cc < (rr < 32 ? 32 : 64)) {
            E* bb = reinterpret_cast<E*>(smem + (which ? SM::oBuf1 : SM::oBuf0));
            bb[(BL::oP >> 1) + BL::tp(rr, cc)] = (E)0.f;
            bb[(BL::oTm >> 1) + BL::tp(rr, cc)] = (E)0.f;
        }
    }
    lds_barrier();

    // ================================ prep waves' state ================================
    const int I = wv - 4, r = 16 * I + l16;  // prep: 16-row block and chunk row of this lane
    const int ptid = threadIdx.x - 256;      // prep thread index 0..255
    unsigned sync_target = 0u;
    Raw8<BF16> rq[NKS], rk[NKS], rb[NKS], ra[NKS];
    float ras_raw = 1.f, rbs_raw = 0.f;
    // (an opaque lane index here too, so that the row addresses are not hoisted out of the loop)
    auto opaque_lane = [&]() __attribute__((always_inline)) {
        int x = lane;
        asm volatile("" : "+v"(x));
        return x;
    };
    auto row_tok = [&](int m, int ln) __attribute__((always_inline)) {  // token index of this lane's row of chunk m (row 0 past the end)
        const int t = m * CH + 16 * I + (ln & 15);
        return (tbase + (t < T ? t : 0)) * H + hh;
    };
    auto load_alpha = [&](int m) __attribute__((always_inline)) {
        const int ln = opaque_lane(), g = ln >> 4;
        const long tok = row_tok(m, ln);
        if constexpr (AS) {
            ras_raw = load_one<BF16>(alpha, tok);
        } else {
#pragma unroll
            for (int s = 0; s < NKS; ++s) ra[s] = gload8<BF16>(alpha, tok * DK + 32 * s + 8 * g);
        }
    };
    // q, k, b through buffer resources over chunk m's rows (rebased per chunk): rows past the end
    // read as zeros
    auto load_qkb = [&](int m) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs_q = rows_rsrc(q, tbase, (long)m * CH, T, (unsigned)(H * DK * 2), CH);
        const __amdgpu_buffer_rsrc_t rs_k = rows_rsrc(k, tbase, (long)m * CH, T, (unsigned)(H * DK * 2), CH);
        const __amdgpu_buffer_rsrc_t rs_b = rows_rsrc(b, tbase, (long)m * CH, T, (unsigned)(H * (BS ? 1 : DK) * 2), CH);
        const int ln = opaque_lane(), g = ln >> 4;
        const unsigned row = (unsigned)(16 * I + (ln & 15)) * H + hh;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int off = (int)((row * DK + 32 * s + 8 * g) * 2u);
            rq[s].u[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_q, off, 0, 0));
            rk[s].u[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_k, off, 0, 0));
            if constexpr (!BS) rb[s].u[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_b, off, 0, 0));
        }
        if constexpr (BS) rbs_raw = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs_b, (int)(row * 2u), 0, 0));
    };

    // Build chunk m's block in `buf` (prep waves only). The raw rows of chunk m are in registers;
    // the loads of chunk m + 1 are issued as soon as the registers free up.
    auto prep_chunk = [&](int m, char* buf) __attribute__((always_inline)) {
        // The lane's row and channel offsets, recomputed from an opaque copy of the lane index in
        // every chunk: otherwise the compiler hoists the many per-lane LDS addresses of this body
        // out of the chunk loop and keeps them all live across it, which spills registers.
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int l16 = lane_o & 15, g = lane_o >> 4, r = 16 * I + l16;
        const int ptid = 64 * I + lane_o;
        E* Qhb = reinterpret_cast<E*>(buf + BL::oQh);
        E* Enb = reinterpret_cast<E*>(buf + BL::oEn);
        E* KbT = reinterpret_cast<E*>(buf + BL::oKbT);
        E* Pm = reinterpret_cast<E*>(buf + BL::oP);
        E* Tm = reinterpret_cast<E*>(buf + BL::oTm);
        E* Kt = reinterpret_cast<E*>(sps + (SM::oKt - SM::oTot));
        E* A16 = reinterpret_cast<E*>(sps + (SM::oA - SM::oTot));
        const bool more = m + 1 < nch;
        const int t = m * CH + r;
        const bool valid = t < T;

        // ---- A: log2-decay of this lane's row and its in-block scan ----
        float lg[CPL];
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
            for (int s = 0; s < NKS; ++s) unpack8<BF16>(keep_or<BF16>(ra[s], valid, GL ? INFINITY : 1.f), &lg[8 * s]);
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
        if (l16 == 15) {
            float* dst = ldsTot + I * DK;
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                float4* p = reinterpret_cast<float4*>(dst + 32 * s + 8 * g);
                p[0] = make_float4(lg[8 * s], lg[8 * s + 1], lg[8 * s + 2], lg[8 * s + 3]);
                p[1] = make_float4(lg[8 * s + 4], lg[8 * s + 5], lg[8 * s + 6], lg[8 * s + 7]);
            }
        }
        prep_sync(ctr, sync_target, lane);

        // ---- decay tables (FusedSmem::kTab) ----
        {
            constexpr int TPC = 256 / DK;
            const int c = ptid % DK, part = ptid / DK;
            float tot[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) tot[J] = ldsTot[J * DK + c];
            const float G[5] = {0.f, tot[0], tot[0] + tot[1], tot[0] + tot[1] + tot[2],
                                tot[0] + tot[1] + tot[2] + tot[3]};
            float e[SM::kTab];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                e[J] = tot[J];
                e[4 + J] = G[J];
                e[8 + J] = G[4] - G[J + 1];
            }
            e[12] = G[4];
            e[13] = tot[1];
            e[14] = tot[1] + tot[2];
            e[15] = tot[2];
#pragma unroll
            for (int tt = 0; tt < SM::kTab; ++tt)
                if (tt % TPC == part) tab[tt * DK + c] = ex2(e[tt]);
        }
        prep_sync(ctr, sync_target, lane);

        // ---- B: factors; K_bar^T and the diagonal P blocks into the block; Q_hat, -E_hat kept ----
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
        // q, k (normalised) and b of 8 channels of this lane's row for K-step s, from raw rows
        auto row_gates = [&](const Raw8<BF16>& rqs, const Raw8<BF16>& rks, const Raw8<BF16>& rbs, float rbsc,
                             float* qx, float* kx, float* bx) __attribute__((always_inline)) {
            unpack8<BF16>(keep_or<BF16>(rqs, valid, 0.f), qx);
            unpack8<BF16>(keep_or<BF16>(rks, valid, 0.f), kx);
            if constexpr (L2N) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    qx[i] *= nq;
                    kx[i] *= nk;
                }
            }
            if constexpr (BS) {
                const float be = GL ? sigmoidf_(rbsc) : rbsc;
#pragma unroll
                for (int i = 0; i < 8; ++i) bx[i] = valid ? be : 0.f;
            } else {
                unpack8<BF16>(keep_or<BF16>(rbs, valid, GL ? -INFINITY : 0.f), bx);
                if constexpr (GL) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) bx[i] = sigmoidf_(bx[i]);
                }
            }
        };
        float er[CPL], qr[CPL];
        float beta_row = 0.f;
        {
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int c0 = 32 * s + 8 * g;
                float qx[8], kx[8], bx[8], fT[8], fG[8], fCG[8];
                row_gates(rq[s], rk[s], rb[s], rbs_raw, qx, kx, bx);
                if (s == 0) beta_row = bx[0];
                lds_read8f(tab + (0 + I) * DK + c0, fT);
                lds_read8f(tab + (4 + I) * DK + c0, fG);
                lds_read8f(tab + (8 + I) * DK + c0, fCG);
                // every factor referenced to the block's first row: fl = 2^lg <= 1 (lg, the scan
                // from the block's start, is <= 0) and its inverse for the column side of the
                // diagonal block, which exceeds fp16 only when the decay across the block's rows
                // passes 2^16 (then the block is redone below)
                float ki[8], kt[8], qh[8], en[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float fl = ex2(lg[8 * s + i]), fli = ex2(-lg[8 * s + i]);
                    const float bk = bx[i] * kx[i];
                    er[8 * s + i] = bk * fl;
                    qr[8 * s + i] = qx[i] * fl;
                    ki[i] = kx[i] * fli;
                    kt[i] = ki[i] * fT[i];
                    qh[i] = qr[8 * s + i] * fG[i];
                    en[i] = -(er[8 * s + i] * fG[i]);
                    KbT[BL::kbt(c0 + i, r)] = (E)(kt[i] * fCG[i]);
                }
                {
                    const Frag kif = PR::make(ki);
                    PR::mma(accA, PR::make(&er[8 * s]), kif);
                    PR::mma(accP, PR::make(&qr[8 * s]), kif);
                }
                put8_units<BL>(Qhb, r, c0, qh);
                put8_units<BL>(Enb, r, c0, en);
                if (I < 3) PR::store8(&Kt[SM::kt(r, c0)], kt);
            }
            bool finite = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) finite = finite && __builtin_isfinite(accA[j]) && __builtin_isfinite(accP[j]);
            if (!__all(finite)) {
                // Strong decay inside the block: redo the diagonal block with bf16 hi/lo operands
                // (a rare path, kept out of line so that it does not add to the main path's registers)
                const DiagPair dp = diag_gram_wide<DK, AS, BS, PRO>(q, k, alpha, b, row_tok(m, lane_o), valid, nq, nk,
                                                                    lane_o);
                accA = dp.a;
                accP = dp.p;
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
        // the next chunk's alpha rows: issued after the factors, the part of this chunk with the
        // most values live (phase A of the next chunk is the first to read them)
        if (more) load_alpha(m + 1);
        prep_sync(ctr, sync_target, lane);

        // ---- C: Gram blocks below the diagonal (wave I: blocks (I, J < I) of A and P); T_II ----
        auto gram_blocks = [&](auto nb_c, const float* c0tab, const float* c1tab) __attribute__((always_inline)) {
            constexpr int NB = decltype(nb_c)::value;
            f4 aA[NB], aP[NB];
#pragma unroll
            for (int J = 0; J < NB; ++J) aA[J] = aP[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int c0 = 32 * s + 8 * g;
                float c8[2][8];
                if constexpr (NB >= 2) lds_read8f(c0tab + c0, c8[0]);
                if constexpr (NB >= 3) lds_read8f(c1tab + c0, c8[1]);
                Frag kf[NB];
#pragma unroll
                for (int J = 0; J < NB; ++J) kf[J] = PR::lds8(Kt + SM::kt(16 * J + l16, c0));
#pragma unroll
                for (int J = 0; J < NB; ++J) {
                    float ea[8], qa[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float f = (J == NB - 1) ? 1.f : c8[J][i];
                        ea[i] = er[8 * s + i] * f;
                        qa[i] = qr[8 * s + i] * f;
                    }
                    PR::mma(aA[J], PR::make(ea), kf[J]);
                    PR::mma(aP[J], PR::make(qa), kf[J]);
                }
            }
#pragma unroll
            for (int J = 0; J < NB; ++J) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 16 * I + 4 * g + j;
                    A16[SM::ar(rr, 16 * J + l16)] = (E)aA[J][j];
                    Pm[BL::tp(rr, 16 * J + l16)] = (E)aP[J][j];
                }
            }
        };
        if (I == 1) {
            gram_blocks(std::integral_constant<int, 1>{}, nullptr, nullptr);
        } else if (I == 2) {
            gram_blocks(std::integral_constant<int, 2>{}, tab + 13 * DK, nullptr);
        } else if (I == 3) {
            gram_blocks(std::integral_constant<int, 3>{}, tab + 14 * DK, tab + 15 * DK);
        } else {
            // T_II = (I + A_II)^-1 for the four diagonal blocks, right-looking: lane group g
            // solves block g, lane l16 owns column l16
            const int Ib = g;
            float acc[16], tc[16];
#pragma unroll
            for (int mm = 0; mm < 16; ++mm) acc[mm] = 0.f;
            const float4* Ab4 = reinterpret_cast<const float4*>(AdT + Ib * SM::ADS);
            float4 cur[4], nxt[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) cur[q4] = Ab4[q4];
#pragma unroll
            for (int mm = 0; mm < 16; ++mm) {
                if (mm + 1 < 16) {
#pragma unroll
                    for (int q4 = (mm + 2) / 4; q4 < 4; ++q4) nxt[q4] = Ab4[(mm + 1) * 4 + q4];
                }
                const float tm = mm < l16 ? 0.f : (mm == l16 ? 1.f : -acc[mm]);
                tc[mm] = tm;
#pragma unroll
                for (int q4 = (mm + 1) / 4; q4 < 4; ++q4) {
                    const float av[4] = {cur[q4].x, cur[q4].y, cur[q4].z, cur[q4].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * q4 + i > mm) acc[4 * q4 + i] = fmaf(av[i], tm, acc[4 * q4 + i]);
                }
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
            }
#pragma unroll
            for (int mm = 0; mm < 16; ++mm) Tm[BL::tp(16 * Ib + mm, 16 * Ib + l16)] = (E)tc[mm];
        }
        prep_sync(ctr, sync_target, lane);

        // the next chunk's q, k, b rows (their registers, and those of this chunk's Gram factors,
        // are free now; phase B of the next chunk is the first to read them)
        if (more) load_qkb(m + 1);

        // ---- D: T10 = -T11 A10 T00 and T32 = -T33 A32 T22 ----
        if (I == 1 || I == 3) {
            const int Ib = I, Jb = I - 1;
            float af[8], bf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = (float)A16[SM::ar(16 * Ib + l16, 16 * Jb + 4 * g + i)];
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
        prep_sync(ctr, sync_target, lane);

        // ---- E: T[32:, :32] = -T[32:, 32:] A[32:, :32] T[:32, :32] ----
        if (I < 2) {
            const int Jb = I;
            f4 Yt[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int Ib = 2 + u;
                const int ra_ = 16 * Ib + l16;
                float bf[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) bf[i] = (float)Tm[BL::tp(kap(g, i), 16 * Jb + l16)];
                Yt[u] = f4{0.f, 0.f, 0.f, 0.f};
                PR::mma(Yt[u], PR::lds_pair(A16 + SM::ar(ra_, 4 * g), A16 + SM::ar(ra_, 16 + 4 * g)), PR::make(bf));
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
        prep_sync(ctr, sync_target, lane);

        // ---- out: gamma_last, beta ----
        float* gc = reinterpret_cast<float*>(buf + BL::oGC);
        if (ptid < DK) gc[ptid] = tab[12 * DK + ptid];
        if constexpr (BS) {
            if (g == 0) reinterpret_cast<float*>(buf + BL::oBeta)[r] = beta_row;
        }
    };

    // ================================ chain waves' state ================================
    const int col0 = tile * DVT + (chain ? wv : 0) * 16;
    const unsigned o_lane = (((unsigned)l16 * H + hh) * DV + col0 + 4 * g) * 4u;
    const unsigned o_tok = (unsigned)H * DV * 4u;
    f4 Sacc[NMK];
    int esc = 0;  // the state is held times sc = 2^esc (rescale_state)
    float sc = 1.f, isc = 1.f;
    const float* s_in = S0 ? S0 + (long)bh * DK * DV : nullptr;
#pragma unroll
    for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sacc[mk][j] = (chain && s_in) ? s_in[(long)(16 * mk + 4 * g + j) * DV + col0 + l16] : 0.f;
    // v, w of this wave's 16 columns for one chunk, straight into registers in the accumulator
    // layout (rows 16 mt + 4 g + j, column col0 + l16), through buffer resources over chunk n's
    // rows (rebased per chunk): rows past the end arrive as zeros
    uint16_t vr[16], wr[16];
    auto load_vw = [&](int n) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs_v = rows_rsrc(v, tbase, (long)n * CH, T, (unsigned)(H * DV * 2), CH);
        const __amdgpu_buffer_rsrc_t rs_w = rows_rsrc(BS ? v : w, tbase, (long)n * CH, T, (unsigned)(H * DV * 2), CH);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned row = (unsigned)(16 * mt + 4 * g + j);
                const int off = (int)(((row * H + hh) * DV + (unsigned)col0 + l16) * 2u);
                vr[4 * mt + j] = __builtin_amdgcn_raw_buffer_load_b16(rs_v, off, 0, 0);
                if constexpr (!BS) wr[4 * mt + j] = __builtin_amdgcn_raw_buffer_load_b16(rs_w, off, 0, 0);
            }
    };
    auto raw_f = [](uint16_t x) __attribute__((always_inline)) { return __uint_as_float((uint32_t)x << 16); };
    auto stack = [](const f4& lo, const f4& hi) __attribute__((always_inline)) {
        float t8[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t8[i] = lo[i];
            t8[i + 4] = hi[i];
        }
        return PR::make(t8);
    };

    // ============ the two roles: the same number of workgroup barriers (1 + chunks) ============
    if (prep) {
        load_alpha(0);
        load_qkb(0);
        prep_chunk(0, smem + SM::oBuf0);
        lds_barrier();
        for (int n = 0; n < nch; ++n) {
            if (n + 1 < nch) prep_chunk(n + 1, smem + (((n + 1) & 1) ? SM::oBuf1 : SM::oBuf0));
            lds_barrier();  // chunk n's buffer is free again; chunk n + 1's is complete
        }
        return;
    }
    if (!chain) {  // (no idle waves at the supported sizes: d_v tiles of 64 columns, 4 chain waves)
        for (int n = 0; n <= nch; ++n) lds_barrier();
        return;
    }
    load_vw(0);
    lds_barrier();
    for (int n = 0; n < nch; ++n) {
        const char* buf = smem + ((n & 1) ? SM::oBuf1 : SM::oBuf0);
        const E* Qh = reinterpret_cast<const E*>(buf + BL::oQh);
        const E* En = reinterpret_cast<const E*>(buf + BL::oEn);
        const E* KbT = reinterpret_cast<const E*>(buf + BL::oKbT);
        const E* Pm = reinterpret_cast<const E*>(buf + BL::oP);
        const E* Tm = reinterpret_cast<const E*>(buf + BL::oTm);
        const float* gC = reinterpret_cast<const float*>(buf + BL::oGC);
        const float* betaL = reinterpret_cast<const float*>(buf + BL::oBeta);
        f4 D[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * mt + 4 * g + j;
                float ww = BS ? betaL[row] : raw_f(wr[4 * mt + j]);
                if constexpr (GL && !BS) ww = sigmoidf_(ww);
                D[mt][j] = ww * raw_f(vr[4 * mt + j]);
            }
        rescale_state<NMK>(Sacc, D, esc, sc, isc);
        float4 gcv[NMK];
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk) gcv[mk] = *reinterpret_cast<const float4*>(gC + 16 * mk + 4 * g);
        __builtin_amdgcn_sched_barrier(0);
        Frag Sf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) Sf[s] = stack(Sacc[2 * s], Sacc[2 * s + 1]);
        // D' = U - E_hat S ; O^T = S^T Q_hat^T
        f4 O[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            O[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int rw = 16 * mt + l16;
                const Frag ef = PR::lds_pair(En + BL::en(rw, 32 * s + 4 * g), En + BL::en(rw, 32 * s + 16 + 4 * g));
                PR::mma(D[mt], ef, Sf[s]);
                const Frag qf = PR::lds_pair(Qh + BL::en(rw, 32 * s + 4 * g), Qh + BL::en(rw, 32 * s + 16 + 4 * g));
                PR::mma(O[mt], Sf[s], qf);
            }
        }
        fused_lookahead<8 * NKS, 6, 1>();
        if (n + 1 < nch) load_vw(n + 1);  // the next chunk's v, w (this chunk's are in D)
        // Delta = T D'
        Frag Df[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) Df[s2] = stack(D[2 * s2], D[2 * s2 + 1]);
        f4 Dl[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            Dl[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 <= mt / 2; ++s2) {
                const int rw = 16 * mt + l16;
                const Frag tf = PR::lds_pair(Tm + BL::tp(rw, 32 * s2 + 4 * g), Tm + BL::tp(rw, 32 * s2 + 16 + 4 * g));
                PR::mma(Dl[mt], tf, Df[s2]);
            }
        }
        fused_lookahead<6, 4, 1>();
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) Df[s2] = stack(Dl[2 * s2], Dl[2 * s2 + 1]);
        // O^T += Delta^T P^T and S <- Diag(gamma_last) S + K_bar^T Delta
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
            for (int s2 = 0; s2 <= nt / 2; ++s2) {
                const int rw = 16 * nt + l16;
                const Frag pf = PR::lds_pair(Pm + BL::tp(rw, 32 * s2 + 4 * g), Pm + BL::tp(rw, 32 * s2 + 16 + 4 * g));
                PR::mma(O[nt], Df[s2], pf);
            }
        }
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk) {
            Sacc[mk][0] *= gcv[mk].x;
            Sacc[mk][1] *= gcv[mk].y;
            Sacc[mk][2] *= gcv[mk].z;
            Sacc[mk][3] *= gcv[mk].w;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int rw = 16 * mk + l16;
                const Frag kf = PR::lds_pair(KbT + BL::kbt(rw, 32 * s2 + 4 * g), KbT + BL::kbt(rw, 32 * s2 + 16 + 4 * g));
                PR::mma(Sacc[mk], kf, Df[s2]);
            }
        }
        fused_lookahead<6 + 2 * NMK, 6, 1>();
        // o rows of this chunk: four consecutive columns per lane, one 16-byte store each
        const __amdgpu_buffer_rsrc_t rs_o = rows_rsrc(o, tbase, (long)n * CH, T, o_tok, CH);
        const unsigned op = o_lane;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            store4(rs_o, op + 16u * nt * o_tok, O[nt][0] * isc, O[nt][1] * isc, O[nt][2] * isc, O[nt][3] * isc);
        lds_barrier();  // chunk n's buffer is free again; chunk n + 1's is complete
    }

    if (S_out) {
        float* s_out = S_out + (long)bh * DK * DV;
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
            for (int j = 0; j < 4; ++j) s_out[(long)(16 * mk + 4 * g + j) * DV + col0 + l16] = Sacc[mk][j] * isc;
    }
}

template <int DK, bool AS, bool BS, int PRO>
hipError_t launch_fused_t(const ChunkArgs& a, hipStream_t s) {
    constexpr int DVT = FusedSmem<DK>::DVT;
    const int tiles = a.DV / DVT;
    const int groups = (a.B * a.H + 7) / 8;
    hipLaunchKernelGGL((fused_kernel<DK, AS, BS, PRO>), dim3(groups * 8 * tiles), dim3(kFusedThreads), 0, s, a.q,
                       a.k, a.v, a.alpha, a.b, a.w, a.S0, a.o, a.S_out, a.B, a.T, a.H, a.DV);
    return hipGetLastError();
}

template <int DK, int PRO>
hipError_t launch_fused_gates(const ChunkArgs& a, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_fused_t<DK, false, false, PRO>(a, s);
        case 1: return launch_fused_t<DK, true, false, PRO>(a, s);
        case 2: return launch_fused_t<DK, false, true, PRO>(a, s);
        default: return launch_fused_t<DK, true, true, PRO>(a, s);
    }
}

template <int DK>
hipError_t launch_fused_dk(const ChunkArgs& a, hipStream_t s) {
#ifdef GDN2_FUSED_PROBE_ONE
    return launch_fused_t<DK, false, false, 0>(a, s);
#else
    switch ((a.flags >> 2) & 3u) {  // GDN2_QK_L2NORM = 4, GDN2_GATE_LOGITS = 8
        case 0: return launch_fused_gates<DK, 0>(a, s);
        case 1: return launch_fused_gates<DK, 1>(a, s);
        case 2: return launch_fused_gates<DK, 2>(a, s);
        default: return launch_fused_gates<DK, 3>(a, s);
    }
#endif
}

}  // namespace

bool fused_supported(int T, int H, int DK, int DV, bool bf16) {
    if (!bf16 || DK != DV || T < 0) return false;
    return DK == 64 || DK == 128;
}

hipError_t launch_fused(const ChunkArgs& a, hipStream_t s) {
    if (!fused_supported(a.T, a.H, a.DK, a.DV, a.bf16)) return hipErrorNotSupported;
#ifdef GDN2_FUSED_PROBE_ONE
    return launch_fused_dk<128>(a, s);
#else
    return a.DK == 64 ? launch_fused_dk<64>(a, s) : launch_fused_dk<128>(a, s);
#endif
}

}  // namespace gdn2
