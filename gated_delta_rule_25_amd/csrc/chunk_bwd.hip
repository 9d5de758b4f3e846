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
//   3. bwd_contract_kernel: per (b, h, chunk), dP = lower(dO Delta^T) and dT = lower(dDelta D'^T),
//      contracted over the value channels on the matrix cores, then dA = -T^T dT T^T in fp32.
//   4. bwd_key_kernel: per (b, h, chunk, 32 key channels), its channels' dQ_hat = dO S^T,
//      dE_hat = -dD' S^T and dK_bar = Delta G'^T on the matrix cores and dgamma, then the
//      decay-weighted sums XA, XP, Y through block references (no factor above 1), the
//      elementwise terms and the reverse cumulative sum; writes dq, dk, db, dalpha.
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
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// four values as fp16 (8 bytes) at byte offset off
__device__ __forceinline__ void store_h4(__amdgpu_buffer_rsrc_t r, unsigned off, float4 x) {
    const h4 h = {(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, (int)off, 0, 0);
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
    uint16_t* G_save;   // [b*h][nch][DK][DV] fp16: dL/dS at the end of each chunk
    uint16_t* dDl;      // [B, T, H, DV] fp16: dL/dDelta
    uint16_t* dDp;      // [B, T, H, DV] fp16: dL/dD'
    float* dv;
    float* dw;
    float* dS0;  // [B, H, DK, DV] or null
    // scalar beta (BS): w points at the [B, T, H] scalars, and the reverse chain writes per token
    // row and 16-column group the partial sums of dL/dbeta through w, dwp[row][npw]
    float* dwp = nullptr;
    int npw = 0;
    int B, T, H, DV, nch;
    // packed batch (VAR): B sequences, T rows, blocks and saves [h][chunk of the batch] with `ring`
    // slots per head
    VarTab var{};
    long ring = 0;
};

// The reverse chain contracts P, T, K_bar, Q_hat and E_hat over the other index than the forward
// chain does, and reads them straight from the block with the transposing LDS read of gfx950
// (ds_read_b64_tr_b16). Within each group of 16 lanes, lane 4 e + a gives the address of four
// consecutive 16-bit elements, and lane 4 a + c receives element c of what lanes 4 e + a
// (e = 0..3) address. Pointed at rows k0 .. k0 + 3 (by e), columns c0 + 4 a .. c0 + 4 a + 3 of a
// row-major Y, lane i of the group thus receives Y[k0 .. k0 + 3][c0 + i]: four k-consecutive
// elements of row c0 + i of Y^T, half of a matrix-core operand. The block layouts permute whole
// 4-element units only, so each lane's address is an ordinary element address. Two block buffers:
// the next block is copied into one while the other is read.
template <int DK>
struct BwdChainSmem {
    using BL = Blob<DK, true>;
    static constexpr int oBuf0 = 0, oBuf1 = BL::bytes;
    // per wave: 64 rows x 16 columns of fp32 (row stride 20) to turn accumulator tiles into rows
    static constexpr int SR = 20;
    static constexpr int oStg = 2 * BL::bytes;
    static constexpr int bytes = oStg + (DK < 64 ? DK : 64) / 16 * CH * SR * 4;
    static_assert(BL::bytes % 16 == 0 && bytes <= 160 * 1024, "reverse chain LDS");
};

__device__ __forceinline__ h4 lds_read_tr(const _Float16* p) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4* lds_s4;
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)p));
}

// Waves own 16 value columns each. The block of the next (earlier) chunk is copied into LDS while
// the current one is worked on, and the next chunk's dO, v, w rows are loaded into registers at
// the start of each step. Rows go to and from memory 16 bytes per lane
// through a per-wave LDS tile, which keeps a step at 52 vector-memory instructions per wave, few
// enough that the next step's wait leaves this step's stores in flight.
template <int DK>
constexpr int bwd_chain_threads() {
    return ((DK < 64 ? DK : 64) / 16) * 64;
}

// WSIG: w holds pre-activations (the prologue's gate logits): the gate is sigma(w), and dw is
// taken with respect to the pre-activation.
// BS: a scalar beta per token row stands for w (its partial gradients go to io.dwp).
// The reverse chain's copy of a block into LDS, issued so that the compiler does not track it.
// Tracked, it makes the compiler wait for the whole copy at the first LDS access it cannot
// separate from it (in practice right after issuing it, before the staging writes), and at every
// LDS barrier. The kernel waits for its copies itself, by count, before the barrier that starts
// each step; no LDS access the compiler can see touches the block buffer before that.
// The instruction writes no register: only LDS (at M0 + 16 lane) and the vector memory count;
// M0 is an input the compiler sets, and the nop covers the wait a write of M0 needs before it.
__device__ __forceinline__ void dma_flat_untracked(const char* g, char* l, int bytes, int cw, int nw, int lane) {
    for (int off = cw * 1024; off < bytes; off += nw * 1024) {
        if (off + lane * 16 < bytes) {
            const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_ptr_t)(l + off));
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g + off + lane * 16), "{m0}"(m) : "memory");
        }
    }
}

template <int DK, bool WSIG = false, bool VAR = false, bool BS = false>
__global__ void __launch_bounds__(bwd_chain_threads<DK>(), 1) bwd_chain_kernel(const ChainBwdIO io) {
    using PR = Prec<true>;
    using E = _Float16;
    using Frag = PR::Frag;
    using BL = Blob<DK, true>;
    using SM = BwdChainSmem<DK>;
    constexpr int NKS = DK / 32, NMK = DK / 16;
    constexpr int DVT = DK < 64 ? DK : 64;
    constexpr int NW = DVT / 16;  // waves, 16 value columns each
    constexpr int NTH = NW * 64;

    __shared__ __attribute__((aligned(16))) char smem[SM::bytes];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int H = io.H, T = io.T, DV = io.DV, nch = io.nch;
    const int vt = DV / DVT;
    // the vt tiles of one (b, h) sit 8 workgroups apart, on one XCD (workgroups go round the 8
    // XCDs in order), so the second tile's block reads hit that XCD's L2
    const int grp = blockIdx.x / (8 * vt), within = blockIdx.x % (8 * vt);
    int bh = grp * 8 + within % 8;
    const int tile = within / 8;
    if (bh >= io.B * io.H) return;  // (the grid is padded to a multiple of 8 (b, h))
    if constexpr (VAR) bh = io.var.perm[bh / H] * H + bh % H;  // longest sequences first
    const int hh = bh % H, bb = bh / H;
    const int col = tile * DVT + 16 * wv + l16;
    // this sequence: its chunks (slots cbase0 ..), first token row and length
    int nchs, Tq;
    long tbase;
    size_t cbase0;
    if constexpr (VAR) {
        const int cf = io.var.coff[bb];
        nchs = io.var.coff[bb + 1] - cf;
        tbase = io.var.start[bb];
        Tq = io.var.len[bb];
        cbase0 = (size_t)hh * io.ring + cf;
    } else {
        nchs = nch;
        tbase = (long)bb * T;
        Tq = T;
        cbase0 = (size_t)bh * nch;
    }
    auto blob_of = [&](int n) { return io.blobs + (cbase0 + n) * BL::bytes; };

    const long seq = tbase * H;
    const unsigned seq_f32 = (unsigned)Tq * H * DV * 4u;
    const auto rs_dO = make_rsrc(io.dO + seq * DV, seq_f32);
    const auto rs_dDl = make_rsrc(io.dDl + seq * DV, seq_f32 / 2u);
    const auto rs_dDp = make_rsrc(io.dDp + seq * DV, seq_f32 / 2u);
    const auto rs_dv = make_rsrc(io.dv + seq * DV, seq_f32);
    const auto rs_dw = make_rsrc(io.dw + seq * DV, seq_f32);
    const auto rs_v = make_rsrc(static_cast<const uint16_t*>(io.v) + seq * DV, (unsigned)Tq * H * DV * 2u);
    const auto rs_w = BS ? make_rsrc(static_cast<const uint16_t*>(io.w) + seq, (unsigned)Tq * H * 2u)
                         : make_rsrc(static_cast<const uint16_t*>(io.w) + seq * DV, (unsigned)Tq * H * DV * 2u);
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
    // operand fragment of row c0 + l16 of Y^T, k = 32 s + kap(g, .), for a block matrix Y with
    // element (r, c) at Y + at(r, c): transposing reads of rows 32 s + 4 g + e and
    // 32 s + 16 + 4 g + e (e = l16 / 4), columns c0 + 4 (l16 % 4) .. + 3
    const int te = l16 >> 2, ta = 4 * (l16 & 3);
    auto frag_t = [&](const E* Y, auto at, int c0, int s) {
        const h4 lo = lds_read_tr(Y + at(32 * s + 4 * g + te, c0 + ta));
        const h4 hi = lds_read_tr(Y + at(32 * s + 16 + 4 * g + te, c0 + ta));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    const auto at_en = [](int r, int c) { return BL::en(r, c); };
    const auto at_kbt = [](int r, int c) { return BL::kbt(r, c); };
    const auto at_tp = [](int r, int c) { return BL::tp(r, c); };

    // Rows as lanes move them: lane (rr = lane / 4 + 16 q, cc = lane % 4), q = 0..3, holds
    // columns 4 cc .. 4 cc + 3 of this wave's 16 at chunk row rr.
    const int rr0 = lane >> 2, cc = lane & 3;
    const int colw = tile * DVT + 16 * wv;  // this wave's first column
    float* stg = reinterpret_cast<float*>(smem + SM::oStg) + wv * CH * SM::SR;
    auto row_off = [&](int row) -> unsigned { return (((unsigned)row * H + hh) * DV + colw + 4 * cc) * 4u; };
    // accumulator tiles (rows 16 mt + 4 g + j, column l16; mt < NT) into the staging tile
    auto stage = [&](const f4* X, auto NTc) {
        constexpr int NT = decltype(NTc)::value;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) stg[(16 * mt + 4 * g + j) * SM::SR + l16] = X[mt][j];
    };
    auto staged = [&](int q) { return *reinterpret_cast<const float4*>(stg + (rr0 + 16 * q) * SM::SR + 4 * cc); };

    // the next chunk's rows: dO (fp32), v and w (bf16), 16 bytes / 8 bytes per lane and row
    u32x4 xdO[4];
    uint32_t xv[4][2], xw[4][2];
    auto fetch = [&](int n) {
        const int t0 = n * CH;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = t0 + rr0 + 16 * q;
            xdO[q] = __builtin_amdgcn_raw_buffer_load_b128(rs_dO, (int)row_off(row), 0, 0);
            const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rs_v, (int)(row_off(row) / 2u), 0, 0);
            xv[q][0] = v2[0];
            xv[q][1] = v2[1];
            if constexpr (BS) {  // the row's scalar beta, as loaded (widened where it is used)
                xw[q][0] = __builtin_amdgcn_raw_buffer_load_b16(rs_w, (int)(((unsigned)row * H + hh) * 2u), 0, 0);
            } else {
                const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(rs_w, (int)(row_off(row) / 2u), 0, 0);
                xw[q][0] = w2[0];
                xw[q][1] = w2[1];
            }
        }
    };
    auto bf = [](uint32_t x, int h) { return __uint_as_float(h ? (x & 0xffff0000u) : (x << 16)); };
    // G (rows 0 .. DK-1 of this wave's 16 columns) to [DK][DV] rows at dst, 64 rows at a time:
    // one 16-byte store per lane and 16 rows
    constexpr int NST = NMK < 4 ? NMK : 4;  // 16-row tiles per round
    auto store_state = [&](float* dst) {
#pragma unroll
        for (int h2 = 0; h2 < NMK / NST; ++h2) {
            stage(&G[NST * h2], std::integral_constant<int, NST>());
#pragma unroll
            for (int q = 0; q < NST; ++q)
                *reinterpret_cast<float4*>(dst + (size_t)(64 * h2 + rr0 + 16 * q) * DV + colw + 4 * cc) = staged(q);
        }
    };
    // the same as fp16 (the G' saves): one 8-byte store per lane and 16 rows
    auto store_state_h = [&](uint16_t* dst) {
#pragma unroll
        for (int h2 = 0; h2 < NMK / NST; ++h2) {
            stage(&G[NST * h2], std::integral_constant<int, NST>());
#pragma unroll
            for (int q = 0; q < NST; ++q) {
                const float4 x = staged(q);
                *reinterpret_cast<h4*>(dst + (size_t)(64 * h2 + rr0 + 16 * q) * DV + colw + 4 * cc) =
                    h4{(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
            }
        }
    };
    // stores a step issues after its loads, whatever the rows: the dD', Delta and dv (and dw) rows;
    // a scalar beta's partial sums are stored only where rows exist, so they are not counted
    constexpr int kStepStores = BS ? 12 : 16;

    if (nchs > 0) {
        dma_flat_untracked(blob_of(nchs - 1), smem + SM::oBuf0, BL::bytes, wv, NW, lane);
        fetch(nchs - 1);
    }
    // (the first step's wait, outside the loop: a wait under a branch in the loop leaves the
    // compiler a path without it, and it then waits again, for everything, at the first use)
    wait_dma();

    for (int idx = 0; idx < nchs; ++idx) {
        const int n = nchs - 1 - idx, t0 = n * CH;
        // block n and this wave's rows of chunk n have arrived (the previous step's stores,
        // issued after them, may still be in flight)
        wait_vm_but<kStepStores>();
        lds_barrier();  // block n is whole; every read of the other buffer (the previous step's) is done
        const char* blk = smem + ((idx & 1) ? SM::oBuf1 : SM::oBuf0);
        const E* En = reinterpret_cast<const E*>(blk + BL::oEn);
        const E* KbT = reinterpret_cast<const E*>(blk + BL::oKbT);
        const E* Tm = reinterpret_cast<const E*>(blk + BL::oTm);
        const E* Pm = reinterpret_cast<const E*>(blk + BL::oP);
        const E* Qh = reinterpret_cast<const E*>(blk + BL::oQh);
        const float* gC = reinterpret_cast<const float*>(blk + BL::oGC);
        // G' of this chunk, for the contraction kernel: stored before this step's loads are
        // issued, so that its staging reads wait for nothing in flight
        store_state_h(io.G_save + (cbase0 + n) * DK * DV);
        if (n > 0) dma_flat_untracked(blob_of(n - 1), smem + ((idx & 1) ? SM::oBuf0 : SM::oBuf1), BL::bytes, wv, NW, lane);

        // this chunk's rows: dO into operand fragments (k = token row 32 s2 + kap(g, i)) through
        // the staging tile; v, w kept for dv, dw; then the loads for the next chunk
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4*>(stg + (rr0 + 16 * q) * SM::SR + 4 * cc) = xdO[q];
        Frag dOf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = stg[(32 * s2 + kap(g, i)) * SM::SR + l16];
            dOf[s2] = PR::make(x);
        }
        float cv[4][4], cw[4][4], cs[4][4];  // v, the gate w, and the factor dw takes
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cv[q][e] = bf(xv[q][e >> 1], e & 1);
                cw[q][e] = BS ? __uint_as_float(xw[q][0] << 16) : bf(xw[q][e >> 1], e & 1);
                cs[q][e] = 1.f;
                if constexpr (WSIG) {
                    cw[q][e] = sigmoidf_(cw[q][e]);
                    cs[q][e] = cw[q][e] * (1.f - cw[q][e]);
                }
            }
        if (n > 0) fetch(n - 1);

        Frag Gf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) Gf[s] = stack(G[2 * s], G[2 * s + 1]);

        // dDelta = P^T dO + K_bar G'   (P^T[m][s] = P[s][m] is zero for s < m)
        f4 dL[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            dL[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = mt / 2; s2 < 2; ++s2) PR::mma(dL[mt], frag_t(Pm, at_tp, 16 * mt, s2), dOf[s2]);
#pragma unroll
            for (int s = 0; s < NKS; ++s) PR::mma(dL[mt], frag_t(KbT, at_kbt, 16 * mt, s), Gf[s]);
        }
        // dD' = T^T dDelta
        const Frag dLf[2] = {stack(dL[0], dL[1]), stack(dL[2], dL[3])};
        f4 dP[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            dP[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = mt / 2; s2 < 2; ++s2) PR::mma(dP[mt], frag_t(Tm, at_tp, 16 * mt, s2), dLf[s2]);
        }
        // rows of dDelta and dD'; dv = w dD', dw = v dD' (rows past T are dropped)
        stage(dL, std::integral_constant<int, 4>());
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x = staged(q);
            store_h4(rs_dDl, row_off(t0 + rr0 + 16 * q) / 2u, x);
        }
        stage(dP, std::integral_constant<int, 4>());
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x = staged(q);
            const unsigned off = row_off(t0 + rr0 + 16 * q);
            store_h4(rs_dDp, off / 2u, x);
            store4<kStreamStore>(rs_dv, off, cw[q][0] * x.x, cw[q][1] * x.y, cw[q][2] * x.z, cw[q][3] * x.w);
            if constexpr (BS) {
                // this row's sum over the wave's 16 columns (the four lanes of the row), one
                // partial per row and 16-column group
                float p = cs[q][0] * (cv[q][0] * x.x + cv[q][1] * x.y + cv[q][2] * x.z + cv[q][3] * x.w);
                p += __shfl_xor(p, 1);
                p += __shfl_xor(p, 2);
                const int t = t0 + rr0 + 16 * q;
                if (cc == 0 && t < Tq) io.dwp[((tbase + t) * H + hh) * io.npw + colw / 16] = p;
            } else {
                store4<kStreamStore>(rs_dw, off, cs[q][0] * cv[q][0] * x.x, cs[q][1] * cv[q][1] * x.y, cs[q][2] * cv[q][2] * x.z,
                       cs[q][3] * cv[q][3] * x.w);
            }
        }
        // dL/dS at the chunk start = Q_hat^T dO + Diag(gamma) G' - E_hat^T dD'  (the block holds -E_hat)
        const Frag dPf[2] = {stack(dP[0], dP[1]), stack(dP[2], dP[3])};
#pragma unroll
        for (int mk = 0; mk < NMK; ++mk) {
            const float4 gm = *reinterpret_cast<const float4*>(gC + 16 * mk + 4 * g);
            G[mk][0] *= gm.x;
            G[mk][1] *= gm.y;
            G[mk][2] *= gm.z;
            G[mk][3] *= gm.w;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                PR::mma(G[mk], frag_t(Qh, at_en, 16 * mk, s2), dOf[s2]);
                PR::mma(G[mk], frag_t(En, at_en, 16 * mk, s2), dPf[s2]);
            }
        }
    }
    if (io.dS0) store_state(io.dS0 + (size_t)bh * DK * DV);
}

// ------------------------------------------------------------------------------------------
// 3. contractions over the value channels, per (b, h, chunk)
struct ContractIO {
    const float* dO;   // [B, T, H, DV]
    const uint16_t* Dp;   // D' (fp16 bits, [B, T, H, DV])
    const uint16_t* Dl;   // Delta
    const uint16_t* dDl;  // dDelta
    const char* blobs;
    float* dPm;  // [b*h][nch][64][64]
    float* dAm;
    int B, T, H, DV, nch;
    VarTab var{};  // packed batch: as ChainBwdIO's
    long ring = 0;
};

// The two 64 x 64 products dP = lower(dO Delta^T) and dT = lower(dDelta D'^T) contract over the
// value channels j with both operands row-major in j, the fragment layout of the matrix cores:
// fp16 operands (as in the chains), fp32 accumulation. The value channels are staged in slices of
// 64 columns; wave w owns output rows 16 w .. 16 w + 15. Then dA = -T^T dT T^T in fp32. (The
// products over the key channels, dQ_hat, dE_hat, dK_bar and dgamma, are formed where they are
// used, in the key kernel.)
template <int DK, bool VAR = false>
__global__ void __launch_bounds__(256, 2) bwd_contract_kernel(const ContractIO io) {
    using PR = Prec<true>;
    using E = _Float16;
    using Frag = PR::Frag;
    using BL = Blob<DK, true>;
    constexpr int JS = DK < 64 ? DK : 64;  // value columns per slice (d_v == d_k)
    constexpr int JP = JS + 4;    // row stride (halves): 2 dwords past a multiple of 32 banks
    constexpr int SMB = 4 * CH * JP * 2;  // bytes of one slice
    constexpr int TP = CH + 1;
    constexpr int UTB = 3 * CH * TP * 4;  // the UT adjoint reuses the slice buffers
    __shared__ __attribute__((aligned(16))) char lds[SMB > UTB ? SMB : UTB];
    E* dOs = reinterpret_cast<E*>(lds);  // [64][JP]: dO, Delta, dDelta, D'
    E* Dls = dOs + CH * JP;
    E* dDls = Dls + CH * JP;
    E* Dps = dDls + CH * JP;

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int H = io.H, T = io.T, DV = io.DV, nch = io.nch;
    // this workgroup's chunk: its slot cbase, first row t0 in the sequence, the sequence's first
    // token row tbase and length Tq (packed: workgroup x = (chunk of the batch) H + h)
    int hh, n, Tq;
    long tbase;
    size_t cbase;
    if constexpr (VAR) {
        hh = blockIdx.x % H;
        const int gc = blockIdx.x / H;
        if (gc >= io.var.coff[io.var.n]) return;
        const int sq = varlen_seq_of(io.var, gc);
        n = gc - io.var.coff[sq];
        tbase = io.var.start[sq];
        Tq = io.var.len[sq];
        cbase = (size_t)hh * io.ring + gc;
    } else {
        const int bh = blockIdx.x / nch;
        n = blockIdx.x % nch;
        hh = bh % H;
        tbase = (long)(bh / H) * T;
        Tq = T;
        cbase = (size_t)bh * nch + n;
    }
    const int t0 = n * CH;

    // T of the block (4-element units of the stored triangle), loaded now, used at the end
    constexpr int TU = BL::TPE / 4;  // units
    constexpr int TPT = (TU + 255) / 256;
    const uint2* Tunits = reinterpret_cast<const uint2*>(io.blobs + cbase * BL::bytes + BL::oTm);
    uint2 tun[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) tun[u] = (tid + 256 * u < TU) ? Tunits[tid + 256 * u] : make_uint2(0u, 0u);

    f4 aP[4], aT[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) aP[c] = aT[c] = f4{0.f, 0.f, 0.f, 0.f};

    // staging: thread x = tid + 256 u takes row x / (JS / 4), columns 4 (x % (JS / 4)) .. + 3
    // (fp32 dO), or row x / (JS / 8), columns 8 (x % (JS / 8)) .. + 7 (fp16 rows); every load of
    // a slice is issued before the first conversion
    constexpr int NRU = CH * JS / 4 / 256, NRH = CH * JS / 8 / 256;
    static_assert(NRU * 256 == CH * JS / 4 && NRH * 256 == CH * JS / 8, "staging split");
    for (int js = 0; js < DV; js += JS) {
        __syncthreads();
        // dO (fp32) 4 columns per thread; Delta, dDelta, D' (fp16 rows) 8 columns per thread
        const uint16_t* srch[3] = {io.Dl, io.dDl, io.Dp};
        E* dsth[3] = {Dls, dDls, Dps};
        float4 lr[NRU];
        uint4 lh[3][NRH];
#pragma unroll
        for (int u = 0; u < NRU; ++u) {
            const int x = tid + 256 * u, r = x / (JS / 4), j = 4 * (x % (JS / 4));
            const int t = t0 + r;
            const size_t e = ((tbase + (t < Tq ? t : 0)) * H + hh) * DV + js + j;
            lr[u] = *reinterpret_cast<const float4*>(io.dO + e);
        }
#pragma unroll
        for (int u = 0; u < NRH; ++u) {
            const int x = tid + 256 * u, r = x / (JS / 8), j = 8 * (x % (JS / 8));
            const int t = t0 + r;
            const size_t e = ((tbase + (t < Tq ? t : 0)) * H + hh) * DV + js + j;
#pragma unroll
            for (int m = 0; m < 3; ++m) lh[m][u] = *reinterpret_cast<const uint4*>(srch[m] + e);
        }
#pragma unroll
        for (int u = 0; u < NRU; ++u) {
            const int x = tid + 256 * u, r = x / (JS / 4), j = 4 * (x % (JS / 4));
            const float4 a = t0 + r < Tq ? lr[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<h4*>(dOs + r * JP + j) = h4{(E)a.x, (E)a.y, (E)a.z, (E)a.w};
        }
#pragma unroll
        for (int u = 0; u < NRH; ++u) {
            const int x = tid + 256 * u, r = x / (JS / 8), j = 8 * (x % (JS / 8));
            const bool ok = t0 + r < Tq;
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const uint4 a = ok ? lh[m][u] : make_uint4(0u, 0u, 0u, 0u);
                *reinterpret_cast<uint2*>(dsth[m] + r * JP + j) = make_uint2(a.x, a.y);
                *reinterpret_cast<uint2*>(dsth[m] + r * JP + j + 4) = make_uint2(a.z, a.w);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < JS / 32; ++ks) {
            const int c0 = 32 * ks + 4 * g;
            auto frag = [&](const E* M, int row) { return PR::lds_pair(M + row * JP + c0, M + row * JP + c0 + 16); };
            const int r = 16 * wv + l16;
            const Frag fO = frag(dOs, r), fdL = frag(dDls, r);
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
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wv + 4 * g + j, cc = 16 * c + l16;
            io.dPm[(cbase * CH + r) * CH + cc] = (c <= wv && cc <= r) ? aP[c][j] : 0.f;
        }

    // dA = -T^T dT T^T (strictly lower), dT = dDelta D'^T on the lower triangle
    __syncthreads();
    float* Tf = reinterpret_cast<float*>(lds);  // [64][TP] T
    float* Tg = Tf + CH * TP;                    // [64][TP] dT
    float* Xm = Tg + CH * TP;                    // [64][TP] T^T dT
    // T into fp32 rows: unit u of the stored triangle is row r, columns 4 cu .. 4 cu + 3 (the
    // inverse of the unit swizzle); rows 0..31 store columns 0..31, the rest are zero
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int x = tid + 256 * u;
        if (x < TU) {
            const int r = x < 256 ? x / 8 : 32 + (x - 256) / 16;
            const int up = x < 256 ? x % 8 : (x - 256) % 16;  // unit position in the stored row
            const int cu = up ^ (x < 256 ? ((r >> 1) & 7) : (r & 15));
            const h4 h = __builtin_bit_cast(h4, tun[u]);
#pragma unroll
            for (int e = 0; e < 4; ++e) Tf[r * TP + 4 * cu + e] = (float)h[e];
        }
    }
    for (int x = tid; x < 32 * 32; x += 256) Tf[(x / 32) * TP + 32 + x % 32] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wv + 4 * g + j, cc = 16 * c + l16;
            Tg[r * TP + cc] = (c <= wv && cc <= r) ? aT[c][j] : 0.f;
        }
    __syncthreads();
    // X = T^T dT, then dA = -X T^T on the strictly lower triangle, on the matrix cores in fp32
    // (16x16x4 steps): wave wv computes rows 16 wv .. 16 wv + 15 as four 16-column tiles. Lane
    // (l16, g) supplies A[l16][g] and B[g][l16] of a step and receives rows 16 wv + 4 g + v,
    // column l16 of the tile. T and dT are lower triangular, so X's tile (wv, c) sums over
    // k >= 16 max(wv, c) only, and dA's tile c <= wv over k < 16 (c + 1); tiles c > wv are zero.
    for (int c = 0; c < 4; ++c) {
        f4 xt = f4{0.f, 0.f, 0.f, 0.f};
        const int k0 = 4 * (wv > c ? wv : c);
        for (int ks = k0; ks < 16; ++ks) {
            const int m = 4 * ks + g;
            xt = __builtin_amdgcn_mfma_f32_16x16x4f32(Tf[m * TP + 16 * wv + l16], Tg[m * TP + 16 * c + l16], xt, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) Xm[(16 * wv + 4 * g + v) * TP + 16 * c + l16] = xt[v];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        f4 d = f4{0.f, 0.f, 0.f, 0.f};
        if (c <= wv) {
            for (int ks = 0; ks < 4 * (c + 1); ++ks) {
                const int m = 4 * ks + g;
                d = __builtin_amdgcn_mfma_f32_16x16x4f32(Xm[(16 * wv + l16) * TP + m], Tf[(16 * c + l16) * TP + m], d, 0, 0, 0);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * wv + 4 * g + v, cc = 16 * c + l16;
            io.dAm[(cbase * CH + r) * CH + cc] = cc < r ? -d[v] : 0.f;
        }
    }
}

// ------------------------------------------------------------------------------------------
// 4. key side, per (b, h, chunk)
struct KeyIO {
    const void *q, *k, *alpha, *b;  // bf16 [B, T, H, DK]
    const float *rnq, *rnk;         // 1 / max(|q|, 1e-12), 1 / max(|k|, 1e-12) per row (L2 norm)
    const float* dO;                  // [B, T, H, DK] (d_v == d_k)
    const uint16_t *dDp, *Dl;         // dL/dD' and Delta rows (fp16, [B, T, H, DK])
    const uint16_t *S_save, *G_save;  // chunk-start states and chunk-end gradients (fp16)
    const float *dPm, *dAm;           // [slot][64][64]
    float *dq, *dk, *dalpha, *db;  // [B, T, H, DK]
    // scalar gates (AS, BS): alpha and b are [B, T, H]; the kernel writes per token row and
    // channel group the partial sums of the scalar's gradient, dap / dbp [row][DK / 32]
    float *dap = nullptr, *dbp = nullptr;
    int B, T, H, nch;
    VarTab var{};  // packed batch: as ChainBwdIO's
    long ring = 0;
};

// One workgroup per (b, h, chunk, 32 key channels): the decay-weighted sums are independent per
// channel. With G the cumulative log2 decay, a factor 2^(G_r - G_s) between row groups X < Y
// (r in Y, s in X) splits at a row between them into two factors no larger than 1:
//   XA, XP (sum over s in X):  2^(G_r - G_e(X)) * [k_s 2^(G_e(X) - G_s)],   e(X) = last row of X,
//   Y      (sum over r in Y):  [x_r 2^(G_r - G_b(Y))] * 2^(G_b(Y) - G_s),   b(Y) = first row of Y,
// so each group pair's sum is a matrix product over pre-scaled rows (fp32 on the matrix cores)
// followed by one scale per output. This is applied twice: between 16-row blocks, then between
// 4-row sub-blocks inside each diagonal block; inside a 4-row sub-block the factor is taken
// directly (one exp2 per pair).
//
// Wave w takes row block I = w; lane (g, l16) owns rows 16 I + 4 g + j (j = 0..3, sub-block
// 4 I + g) and channels 2 l16 + c (c = 0, 1) of the group, which is the matrix cores' output
// layout when column l16 of tile c stands for channel 2 l16 + c.
// PRO (prologue, as prep_kernel's): bit 0, q and k are normalised here (io.rnq, io.rnk) and dq, dk
// are left with respect to the normalised vectors (a later pass takes them through the norm);
// bit 1, alpha and b are pre-activations: log2 alpha = log2 sigma(x), b = sigma(x), and dalpha, db
// are taken with respect to the pre-activations.
template <int DK, int PRO = 0, bool VAR = false, bool AS = false, bool BS = false>
__global__ void __launch_bounds__(256, 2) bwd_key_kernel(const KeyIO io) {
    constexpr bool L2N = (PRO & 1) != 0, GL = (PRO & 2) != 0;
    constexpr int CW = 32;       // key channels per workgroup
    constexpr int NG = DK / CW;  // channel groups
    static_assert(DK % CW == 0, "channel groups");
    using PR = Prec<true>;
    using E = _Float16;
    using Frag = PR::Frag;
    // LDS: first the staged operands of the contraction over the value channels, then, in the
    // same bytes, the arrays of the decay-weighted sums
    constexpr int JP = DK + 4;  // staged row stride (halves): 2 dwords past a multiple of 32 banks
    constexpr int kStage = (3 * CH + 2 * CW) * JP * 2;
    constexpr int kSums = (2 * CH * CH + 4 * CH * CW + 16 * CW) * 4;
    __shared__ __attribute__((aligned(16))) char smem[kStage > kSums ? kStage : kSums];
    __shared__ float dgS[CW];  // dgamma of the group's channels, by staged row
    float* dA = reinterpret_cast<float*>(smem);
    float* dPs = dA + CH * CH;
    float* G2 = dPs + CH * CH;  // cumulative log2 decay
    float* Xk = G2 + CH * CW;   // pre-scaled rows of k, b*k, q
    float* Xe = Xk + CH * CW;
    float* Xq = Xe + CH * CW;
    float* part = Xq + CH * CW;  // per sub-block sums over rows
    E* Os = reinterpret_cast<E*>(smem);  // [CH][JP] rows of dO, dD', Delta
    E* DPs = Os + CH * JP;
    E* Ls = DPs + CH * JP;
    E* Sg = Ls + CH * JP;  // [CW][JP] the group's rows of S and G': staged row 16 t + l is channel 2 l + t
    E* Gg = Sg + CW * JP;

    const int tid = threadIdx.x, I = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int H = io.H, T = io.T, nch = io.nch;
    // the NG channel groups of one chunk sit 8 workgroups apart, on one XCD (workgroups go round
    // the 8 XCDs in order), so their reads of the chunk's dA and dP share that XCD's L2
    const int w8 = blockIdx.x % 8, rest = blockIdx.x / 8;
    const int cg = rest % NG, item = (rest / NG) * 8 + w8;
    // this workgroup's chunk (as in the contraction kernel; packed: item = (chunk of the batch) H + h)
    int hh, n, Tq;
    long tbase;
    size_t cbase;
    if constexpr (VAR) {
        hh = item % H;
        const int gc = item / H;
        if (gc >= io.var.coff[io.var.n]) return;
        const int sq = varlen_seq_of(io.var, gc);
        n = gc - io.var.coff[sq];
        tbase = io.var.start[sq];
        Tq = io.var.len[sq];
        cbase = (size_t)hh * io.ring + gc;
    } else {
        if (item >= io.B * io.H * io.nch) return;
        const int bh = item / nch;
        n = item % nch;
        hh = bh % H;
        tbase = (long)(bh / H) * T;
        Tq = T;
        cbase = (size_t)bh * nch + n;
    }
    const int t0 = n * CH, c0 = cg * CW;
    const int ch0 = 2 * l16;  // this lane's first channel in the group
    const int rb = 16 * I + 4 * g;  // this lane's first row
    auto lo = [](uint32_t x) { return __uint_as_float(x << 16); };
    auto hi = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };

    // ---- loads, all issued before the first use ----
    const uint32_t* q32 = static_cast<const uint32_t*>(io.q);
    const uint32_t* k32 = static_cast<const uint32_t*>(io.k);
    const uint32_t* a32 = static_cast<const uint32_t*>(io.alpha);
    const uint32_t* b32 = static_cast<const uint32_t*>(io.b);
    uint32_t rq[4], rk[4], rbv[4], ra[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = t0 + rb + j;
        const size_t rowi = (tbase + (t < Tq ? t : 0)) * H + hh;
        const size_t e = (rowi * DK + c0 + ch0) / 2;
        rq[j] = q32[e];
        rk[j] = k32[e];
        // a scalar gate goes in both halves of the word, as if repeated over the channel pair
        if constexpr (BS) {
            const uint32_t x = static_cast<const uint16_t*>(io.b)[rowi];
            rbv[j] = x | (x << 16);
        } else {
            rbv[j] = b32[e];
        }
        if constexpr (AS) {
            const uint32_t x = static_cast<const uint16_t*>(io.alpha)[rowi];
            ra[j] = x | (x << 16);
        } else {
            ra[j] = a32[e];
        }
    }

    // ---- dQ_hat = dO S^T, dE_hat = -dD' S^T, dK_bar = Delta G'^T for this group's channels,
    // contracted over the value channels on the matrix cores (fp16 operands as in the chains,
    // fp32 accumulate), and dgamma = rowsum(S o G') of the group in fp32 from the same values.
    // Thread x = tid + 256 u stages row x / (DK / 4), columns 4 (x % (DK / 4)) .. + 3 of dO, or
    // row x / (DK / 8), columns 8 (x % (DK / 8)) .. + 7 of an fp16 row; rows past the end are
    // read at row 0 and staged as zeros. ----
    constexpr int NO = CH * DK / 4 / 256, NH = CH * DK / 8 / 256;
    constexpr int NSR = CW * DK / 8, NSU = (NSR + 255) / 256;  // S, G' units of 8
    static_assert(NO * 256 == CH * DK / 4 && NH * 256 == CH * DK / 8, "staging split");
    float4 lo4[NO];
    uint4 lh[2][NH], ls[2][NSU];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int x = tid + 256 * u, r = x / (DK / 4), j = 4 * (x % (DK / 4)), t = t0 + r;
        lo4[u] = *reinterpret_cast<const float4*>(io.dO + ((tbase + (t < Tq ? t : 0)) * H + hh) * DK + j);
    }
#pragma unroll
    for (int u = 0; u < NH; ++u) {
        const int x = tid + 256 * u, r = x / (DK / 8), j = 8 * (x % (DK / 8)), t = t0 + r;
        const size_t e = ((tbase + (t < Tq ? t : 0)) * H + hh) * DK + j;
        lh[0][u] = *reinterpret_cast<const uint4*>(io.dDp + e);
        lh[1][u] = *reinterpret_cast<const uint4*>(io.Dl + e);
    }
#pragma unroll
    for (int u = 0; u < NSU; ++u) {
        const int x = tid + 256 * u, sr = x / (DK / 8), j = 8 * (x % (DK / 8));
        ls[0][u] = ls[1][u] = make_uint4(0u, 0u, 0u, 0u);
        if (x < NSR) {
            const size_t e = (cbase * DK + c0 + 2 * (sr % 16) + sr / 16) * DK + j;
            ls[0][u] = *reinterpret_cast<const uint4*>(io.S_save + e);
            ls[1][u] = *reinterpret_cast<const uint4*>(io.G_save + e);
        }
    }
    auto put8 = [&](E* dst, uint4 a) {  // 8 halves at an 8-byte aligned row position
        *reinterpret_cast<uint2*>(dst) = make_uint2(a.x, a.y);
        *reinterpret_cast<uint2*>(dst + 4) = make_uint2(a.z, a.w);
    };
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int x = tid + 256 * u, r = x / (DK / 4), j = 4 * (x % (DK / 4));
        const float4 a = t0 + r < Tq ? lo4[u] : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<h4*>(Os + r * JP + j) = h4{(E)a.x, (E)a.y, (E)a.z, (E)a.w};
    }
#pragma unroll
    for (int u = 0; u < NH; ++u) {
        const int x = tid + 256 * u, r = x / (DK / 8), j = 8 * (x % (DK / 8));
        const bool ok = t0 + r < Tq;
        put8(DPs + r * JP + j, ok ? lh[0][u] : make_uint4(0u, 0u, 0u, 0u));
        put8(Ls + r * JP + j, ok ? lh[1][u] : make_uint4(0u, 0u, 0u, 0u));
    }
#pragma unroll
    for (int u = 0; u < NSU; ++u) {
        const int x = tid + 256 * u, sr = x / (DK / 8), j = 8 * (x % (DK / 8));
        float p = 0.f;
        if (x < NSR) {
            put8(Sg + sr * JP + j, ls[0][u]);
            put8(Gg + sr * JP + j, ls[1][u]);
            const uint32_t sa[4] = {ls[0][u].x, ls[0][u].y, ls[0][u].z, ls[0][u].w};
            const uint32_t ga[4] = {ls[1][u].x, ls[1][u].y, ls[1][u].z, ls[1][u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const E* s2 = reinterpret_cast<const E*>(&sa[e]);
                const E* g2 = reinterpret_cast<const E*>(&ga[e]);
                p = fmaf((float)s2[0], (float)g2[0], p);
                p = fmaf((float)s2[1], (float)g2[1], p);
            }
        }
#pragma unroll
        for (int m = 1; m < DK / 8; m <<= 1) p += __shfl_xor(p, m);  // the row's DK / 8 lanes
        if (x < NSR && x % (DK / 8) == 0) dgS[sr] = p;
    }
    float lA[16], lP[16];  // dA and dP of the chunk, for the sums below
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        lA[u] = io.dAm[cbase * CH * CH + tid + 256 * u];
        lP[u] = io.dPm[cbase * CH * CH + tid + 256 * u];
    }
    __syncthreads();
    f4 aQ[2], aE[2], aK[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) aQ[t] = aE[t] = aK[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const int k0 = 32 * ks + 4 * g;
        auto frag = [&](const E* M, int row) { return PR::lds_pair(M + row * JP + k0, M + row * JP + k0 + 16); };
        const int r = 16 * I + l16;
        const Frag fO = frag(Os, r), fDp = frag(DPs, r), fL = frag(Ls, r);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const Frag fS = frag(Sg, 16 * t + l16), fG = frag(Gg, 16 * t + l16);
            PR::mma(aQ[t], fO, fS);
            PR::mma(aE[t], fDp, fS);
            PR::mma(aK[t], fL, fG);
        }
    }
    __syncthreads();  // the staged operands are read; their bytes are reused below
    // accumulator [t][j]: row 16 I + 4 g + j = rb + j, column l16 of tile t = channel 2 l16 + t
    float2 gQ[4], gE[4], gK[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gQ[j] = make_float2(aQ[0][j], aQ[1][j]);
        gE[j] = make_float2(-aE[0][j], -aE[1][j]);
        gK[j] = make_float2(aK[0][j], aK[1][j]);
    }
    const float2 dgam = make_float2(dgS[l16], dgS[16 + l16]);

    float nq[4] = {1.f, 1.f, 1.f, 1.f}, nk[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (L2N) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + rb + j;
            const size_t row = (tbase + (t < Tq ? t : 0)) * H + hh;
            nq[j] = io.rnq[row];
            nk[j] = io.rnk[row];
        }
    }
    // this lane's inputs; rows past the end read as zero and do not decay
    float q[4][2], k[4][2], bb2[4][2], la[4][2], G[4][2];
    auto lg2a = [](float x) { return GL ? lg2_sigmoid(x) : __builtin_amdgcn_logf(x); };
    auto gate = [](float x) { return GL ? sigmoidf_(x) : x; };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool ok = t0 + rb + j < Tq;
        q[j][0] = ok ? lo(rq[j]) * nq[j] : 0.f;
        q[j][1] = ok ? hi(rq[j]) * nq[j] : 0.f;
        k[j][0] = ok ? lo(rk[j]) * nk[j] : 0.f;
        k[j][1] = ok ? hi(rk[j]) * nk[j] : 0.f;
        bb2[j][0] = ok ? gate(lo(rbv[j])) : 0.f;
        bb2[j][1] = ok ? gate(hi(rbv[j])) : 0.f;
        la[j][0] = ok ? lg2a(lo(ra[j])) : 0.f;
        la[j][1] = ok ? lg2a(hi(ra[j])) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        dA[tid + 256 * u] = lA[u];
        dPs[tid + 256 * u] = lP[u];
    }
    // ---- G: prefix within the sub-block, then the totals of the sub-blocks before it ----
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc += la[j][c];
            G[j][c] = acc;
        }
        part[(4 * I + g) * CW + ch0 + c] = acc;
    }
    __syncthreads();
    {
        // the sub-blocks before this lane's, added in order; every read issued at once
        float pre[2] = {0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < 15; ++sb) {
            const float2 p = *reinterpret_cast<const float2*>(&part[sb * CW + ch0]);
            if (sb < 4 * I + g) {
                pre[0] += p.x;
                pre[1] += p.y;
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                G[j][c] += pre[c];
                G2[(rb + j) * CW + ch0 + c] = G[j][c];
            }
    }
    __syncthreads();

    // ---- rows pre-scaled against this block's ends: k to its last row, b*k and q to its first ----
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float Ge = G2[(16 * I + 15) * CW + ch0 + c], Gb = G2[(16 * I) * CW + ch0 + c];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int x = (rb + j) * CW + ch0 + c;
            const float down = __builtin_amdgcn_exp2f(G[j][c] - Gb);
            Xk[x] = k[j][c] * __builtin_amdgcn_exp2f(Ge - G[j][c]);
            Xe[x] = bb2[j][c] * k[j][c] * down;
            Xq[x] = q[j][c] * down;
        }
    }
    __syncthreads();

    // ---- between 16-row blocks: XA, XP over blocks J < I, Y over blocks I2 > I ----
    f4 xa[2], xp[2], yy[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) xa[c] = xp[c] = yy[c] = f4{0.f, 0.f, 0.f, 0.f};
    for (int J = 0; J < I; ++J) {
        f4 sa[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
        f4 sp[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ip = 0; ip < 4; ++ip) {
            const int s2 = 16 * J + 4 * g + ip;
            const float av = dA[(16 * I + l16) * CH + s2], pv = dPs[(16 * I + l16) * CH + s2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float kv = Xk[s2 * CW + ch0 + c];
                sa[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, kv, sa[c], 0, 0, 0);
                sp[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, kv, sp[c], 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float Ge = G2[(16 * J + 15) * CW + ch0 + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = __builtin_amdgcn_exp2f(G[j][c] - Ge);
                xa[c][j] = fmaf(f, sa[c][j], xa[c][j]);
                xp[c][j] = fmaf(f, sp[c][j], xp[c][j]);
            }
        }
    }
    for (int I2 = I + 1; I2 < 4; ++I2) {
        f4 sy[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ip = 0; ip < 4; ++ip) {
            const int r2 = 16 * I2 + 4 * g + ip;
            const float av = dA[r2 * CH + 16 * I + l16], pv = dPs[r2 * CH + 16 * I + l16];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                sy[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, Xe[r2 * CW + ch0 + c], sy[c], 0, 0, 0);
                sy[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, Xq[r2 * CW + ch0 + c], sy[c], 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float Gb = G2[(16 * I2) * CW + ch0 + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) yy[c][j] = fmaf(__builtin_amdgcn_exp2f(Gb - G[j][c]), sy[c][j], yy[c][j]);
        }
    }
    __syncthreads();  // every read of the block-level rows is done

    // ---- between 4-row sub-blocks inside the diagonal block: the same with sub-block ends ----
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int x = (rb + j) * CW + ch0 + c;
            const float down = __builtin_amdgcn_exp2f(G[j][c] - G[0][c]);
            Xk[x] = k[j][c] * __builtin_amdgcn_exp2f(G[3][c] - G[j][c]);
            Xe[x] = bb2[j][c] * k[j][c] * down;
            Xq[x] = q[j][c] * down;
        }
    // (the rows read below belong to this wave's block: its own writes above come first)
#pragma unroll
    for (int V = 0; V < 3; ++V) {  // XA, XP of rows in sub-blocks g > V
        const int s2 = 16 * I + 4 * V + g;
        const float av = dA[(16 * I + l16) * CH + s2], pv = dPs[(16 * I + l16) * CH + s2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float kv = Xk[s2 * CW + ch0 + c];
            const f4 z = f4{0.f, 0.f, 0.f, 0.f};
            const f4 sa = __builtin_amdgcn_mfma_f32_16x16x4f32(av, kv, z, 0, 0, 0);
            const f4 sp = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, kv, z, 0, 0, 0);
            const float Ge = G2[(16 * I + 4 * V + 3) * CW + ch0 + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = g > V ? __builtin_amdgcn_exp2f(G[j][c] - Ge) : 0.f;
                xa[c][j] = fmaf(f, sa[j], xa[c][j]);
                xp[c][j] = fmaf(f, sp[j], xp[c][j]);
            }
        }
    }
#pragma unroll
    for (int W = 1; W < 4; ++W) {  // Y of rows in sub-blocks g < W
        const int r2 = 16 * I + 4 * W + g;
        const float av = dA[r2 * CH + 16 * I + l16], pv = dPs[r2 * CH + 16 * I + l16];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f4 sy = f4{0.f, 0.f, 0.f, 0.f};
            sy = __builtin_amdgcn_mfma_f32_16x16x4f32(av, Xe[r2 * CW + ch0 + c], sy, 0, 0, 0);
            sy = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, Xq[r2 * CW + ch0 + c], sy, 0, 0, 0);
            const float Gb = G2[(16 * I + 4 * W) * CW + ch0 + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = W > g ? __builtin_amdgcn_exp2f(Gb - G[j][c]) : 0.f;
                yy[c][j] = fmaf(f, sy[j], yy[c][j]);
            }
        }
    }

    // ---- inside this lane's sub-block: pairs j' <= j term by term ----
    float Asb[4][4], Psb[4][4];  // [row j][column j'] of the sub-block's dA and dP
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 x = *reinterpret_cast<const float4*>(&dA[(rb + j) * CH + rb]);
        const float4 y = *reinterpret_cast<const float4*>(&dPs[(rb + j) * CH + rb]);
        Asb[j][0] = x.x; Asb[j][1] = x.y; Asb[j][2] = x.z; Asb[j][3] = x.w;
        Psb[j][0] = y.x; Psb[j][1] = y.y; Psb[j][2] = y.z; Psb[j][3] = y.w;
    }
    const float G63c[2] = {G2[(CH - 1) * CW + ch0], G2[(CH - 1) * CW + ch0 + 1]};
    float dG[4][2], kbs[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float XA[4], XP[4], Y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            XA[j] = xa[c][j];
            XP[j] = fmaf(Psb[j][j], k[j][c], xp[c][j]);
            Y[j] = fmaf(Psb[j][j], q[j][c], yy[c][j]);
        }
#pragma unroll
        for (int j = 1; j < 4; ++j)
#pragma unroll
            for (int jp = 0; jp < j; ++jp) {  // row j, earlier row jp: F = 2^(G_j - G_jp) <= 1
                const float F = __builtin_amdgcn_exp2f(G[j][c] - G[jp][c]);
                XA[j] = fmaf(Asb[j][jp] * F, k[jp][c], XA[j]);
                XP[j] = fmaf(Psb[j][jp] * F, k[jp][c], XP[j]);
                Y[jp] = fmaf(F, fmaf(Asb[j][jp], bb2[j][c] * k[j][c], Psb[j][jp] * q[j][c]), Y[jp]);
            }
        // ---- elementwise: the gradients of q, k, b and dL/dG of each row ----
        kbs[c] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float gq = c ? gQ[j].y : gQ[j].x, ge = c ? gE[j].y : gE[j].x, gk = c ? gK[j].y : gK[j].x;
            const float eG = __builtin_amdgcn_exp2f(G[j][c]), eK = __builtin_amdgcn_exp2f(G63c[c] - G[j][c]);
            const float kr = k[j][c], qr = q[j][c], br = bb2[j][c], Et = br * kr;
            const float dEt = fmaf(ge, eG, XA[j]);
            dG[j][c] = gq * qr * eG + ge * Et * eG - gk * kr * eK + Et * XA[j] + qr * XP[j] - kr * Y[j];
            kbs[c] = fmaf(gk, kr * eK, kbs[c]);
            XA[j] = fmaf(gq, eG, XP[j]);                 // dq
            XP[j] = fmaf(gk, eK, Y[j]) + br * dEt;       // dk
            Y[j] = kr * dEt;                             // db
            if constexpr (GL) Y[j] *= br * (1.f - br);   // with respect to the pre-activation
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // park the outputs of channel c in xa/xp/yy
            xa[c][j] = XA[j];
            xp[c][j] = XP[j];
            yy[c][j] = Y[j];
        }
    }
    // a scalar gate's gradient: the row's sum over the group's 32 channels (the 16 lanes of the
    // row, two channels each), one partial per row and channel group
    auto row_partial = [&](float x) {
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        return x;
    };
    // dq, dk, db, dalpha go out with the streaming store policy (no later kernel reads them),
    // through buffer resources over the chunk's rows (rows past the end are dropped)
    const unsigned gb = (unsigned)(H * DK * 4);
    auto stream2 = [&](float* dst, int j, float x, float y) {
        const unsigned off = (unsigned)((((rb + j) * H + hh) * DK + c0 + ch0) * 4);
        const u32x2 v = {__float_as_uint(x), __float_as_uint(y)};
        __builtin_amdgcn_raw_buffer_store_b64(v, rows_rsrc(dst, tbase, t0, Tq, gb, CH), (int)off, 0, kStreamStore);
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = t0 + rb + j;
        float pb = 0.f;
        if constexpr (BS) pb = row_partial(yy[0][j] + yy[1][j]);
        stream2(io.dq, j, xa[0][j], xa[1][j]);
        stream2(io.dk, j, xp[0][j], xp[1][j]);
        if constexpr (BS) {
            if (t < Tq && l16 == 0) io.dbp[((tbase + t) * H + hh) * NG + cg] = pb;
        } else {
            stream2(io.db, j, yy[0][j], yy[1][j]);
        }
    }

    // ---- dlog(alpha)_r = sum over rows r2 >= r of dG_r2; the last row also carries
    // sum_r dK_bar K_bar and dgamma gamma. alpha_r = 2^(la_r). ----
    __syncthreads();  // every read of part is done
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float kb = kbs[c];
        kb += __shfl_xor(kb, 16);
        kb += __shfl_xor(kb, 32);
        part[(4 * I + g) * CW + ch0 + c] = dG[0][c] + dG[1][c] + dG[2][c] + dG[3][c];
        if (g == 0) G2[I * CW + ch0 + c] = kb;  // (G2 is no longer needed: rows 0..3 take the sums)
    }
    __syncthreads();
    float dal[4][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float acc = (c ? dgam.y : dgam.x) * __builtin_amdgcn_exp2f(G63c[c]);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += G2[w * CW + ch0 + c];
        float later[15];  // the sub-blocks after this lane's, added in order; reads issued at once
#pragma unroll
        for (int sb = 1; sb < 16; ++sb) later[sb - 1] = part[sb * CW + ch0 + c];
#pragma unroll
        for (int sb = 1; sb < 16; ++sb)
            if (sb > 4 * I + g) acc += later[sb - 1];
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            acc += dG[j][c];
            // acc = dL/d ln(alpha), alpha = 2^la; d ln sigma(x)/dx = 1 - sigma(x)
            dal[j][c] = GL ? acc * (1.f - __builtin_amdgcn_exp2f(la[j][c])) : acc * __builtin_amdgcn_exp2f(-la[j][c]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = t0 + rb + j;
        float pa = 0.f;
        if constexpr (AS) pa = row_partial(dal[j][0] + dal[j][1]);
        if constexpr (AS) {
            if (t < Tq && l16 == 0) io.dap[((tbase + t) * H + hh) * NG + cg] = pa;
        } else {
            stream2(io.dalpha, j, dal[j][0], dal[j][1]);
        }
    }
}

__global__ void __launch_bounds__(256) copy_or_zero(float* dst, const float* src, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// The gradients of the scalar gates from the kernels' per-row partial sums, added in a fixed
// order: dalpha[r] = sum of dap[r][0 .. na), db[r] = sum of dbp[r][0 .. nb) + sum of dwp[r][0 .. nw).
__global__ void __launch_bounds__(256) scalar_gate_sums(const float* __restrict__ dap, int na,
                                                        const float* __restrict__ dbp, int nb,
                                                        const float* __restrict__ dwp, int nw,
                                                        float* __restrict__ dalpha, float* __restrict__ db, long rows) {
    const long r = (long)blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    if (dap) {
        float x = 0.f;
        for (int i = 0; i < na; ++i) x += dap[r * na + i];
        dalpha[r] = x;
    }
    if (dbp) {
        float x = 0.f;
        for (int i = 0; i < nb; ++i) x += dbp[r * nb + i];
        float y = 0.f;
        for (int i = 0; i < nw; ++i) y += dwp[r * nw + i];
        db[r] = x + y;
    }
}

// 1 / max(|x|, 1e-12) of each row of D bf16 values. A group of D / 8 lanes owns a row, one
// 16-byte load per lane; the row's sum is a butterfly inside the group.
template <int D>
__global__ void __launch_bounds__(256) row_rnorm(const uint16_t* __restrict__ x, float* __restrict__ rn, long rows) {
    constexpr int LPR = D / 8, RPB = 256 / LPR;  // lanes per row, rows per workgroup
    const long r = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = (threadIdx.x % LPR) * 8;
    float ss = 0.f;
    if (r < rows) {  // groups are row-aligned: a group is all in or all out
        const uint4 u = *reinterpret_cast<const uint4*>(x + r * D + c);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (r < rows && threadIdx.x % LPR == 0) rn[r] = 1.f / fmaxf(sqrtf(ss), 1e-12f);
}

// Through the L2 norm, in place: dx (with respect to x_n = x rn) becomes
// rn (dx - (dx . x_n) x_n), or dx rn where |x| <= 1e-12 (rn = 1e12: x_n = x / 1e-12 there).
// A group of D / 4 lanes owns a row: 16 bytes of dx and 8 of x per lane.
template <int D>
__global__ void __launch_bounds__(256) l2norm_bwd(float* __restrict__ dx, const uint16_t* __restrict__ x,
                                                  const float* __restrict__ rn, long rows) {
    constexpr int LPR = D / 4, RPB = 256 / LPR;
    const long r = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = (threadIdx.x % LPR) * 4;
    const bool live = r < rows;
    float4 gv = make_float4(0.f, 0.f, 0.f, 0.f);
    uint2 u = make_uint2(0u, 0u);
    float n = 0.f;
    if (live) {
        gv = *reinterpret_cast<const float4*>(dx + r * D + c);
        u = *reinterpret_cast<const uint2*>(x + r * D + c);
        n = rn[r];
    }
    const float g[4] = {gv.x, gv.y, gv.z, gv.w};
    const float xn[4] = {__uint_as_float(u.x << 16) * n, __uint_as_float(u.x & 0xffff0000u) * n,
                         __uint_as_float(u.y << 16) * n, __uint_as_float(u.y & 0xffff0000u) * n};
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dot = fmaf(g[e], xn[e], dot);
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
    const bool tiny = n >= 1e12f;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = tiny ? g[e] * n : n * fmaf(-dot, xn[e], g[e]);
    if (live) *reinterpret_cast<float4*>(dx + r * D + c) = make_float4(o[0], o[1], o[2], o[3]);
}

struct BwdLayout {
    size_t blobs, S_save, G_save, Dp, Dl, dDl, dDp, dPm, dAm, total;
};

// Workspace of the backward: `head` bytes first (the sequence table of a packed batch), then the
// per-chunk buffers for `slots` chunks (b*h*chunks, or h * chunk bound of a packed batch) and the
// per-row buffers for `tok_rows` token rows (b*t*h).
BwdLayout bwd_layout_n(size_t slots, size_t tok_rows, int DK, int DV, size_t head) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    BwdLayout L{};
    size_t o = up(head);
    L.blobs = o;
    o += up(slots * split_chunk_bytes(1, 1, DK, true));
    const size_t st = up(slots * DK * DV * 2);  // fp16 states
    L.S_save = o;
    o += st;
    L.G_save = o;
    o += st;
    const size_t rows = up(tok_rows * DV * 2);  // fp16 rows
    L.Dp = o;
    o += rows;
    L.Dl = o;
    o += rows;
    L.dDl = o;
    o += rows;
    L.dDp = o;
    o += rows;
    const size_t pm = up(slots * CH * CH * 4);
    L.dPm = o;
    o += pm;
    L.dAm = o;
    o += pm;
    L.total = o;
    return L;
}

BwdLayout bwd_layout(int B, int T, int H, int DK, int DV) {
    const size_t nch = ((size_t)T + CH - 1) / CH;
    return bwd_layout_n((size_t)B * H * nch, (size_t)B * T * H, DK, DV, 0);
}

// packed batch of n sequences, T rows
BwdLayout bwd_layout_var(int n, int T, int H, int DK, int DV) {
    return bwd_layout_n((size_t)H * varlen_chunk_bound(n, T), (size_t)T * H, DK, DV, varlen_table_bytes(n));
}

// Scalar gates (AS, BS): the kernels read the [B, T, H] scalars themselves and write per-row
// partial sums of their gradients into dap (DK / 32 per row), dbp (DK / 32) and dwp (DV / 16);
// scalar_gate_sums adds them up.
template <int DK, int PRO, bool VAR, bool AS, bool BS>
hipError_t launch_bwd_t(const BwdArgs& a, const float* rnq, const float* rnk, float* dap, float* dbp, float* dwp,
                        hipStream_t st) {
    const BwdLayout L = VAR ? bwd_layout_var(a.B, a.T, a.H, DK, a.DV) : bwd_layout(a.B, a.T, a.H, DK, a.DV);
    char* ws = static_cast<char*>(a.workspace);
    const int BH = a.B * a.H, nch = (a.T + CH - 1) / CH;
    const long ring = VAR ? varlen_chunk_bound(a.B, a.T) : 0;  // chunk slots per head (packed)
    VarTab vt;
    if constexpr (VAR) {
        vt.coff = reinterpret_cast<const int*>(ws);
        vt.start = vt.coff + a.B + 1;
        vt.len = vt.start + a.B;
        vt.perm = vt.len + a.B;
        vt.n = a.B;
    }
    char* blobs = ws + L.blobs;
    uint16_t* S_save = reinterpret_cast<uint16_t*>(ws + L.S_save);
    uint16_t* G_save = reinterpret_cast<uint16_t*>(ws + L.G_save);
    uint16_t* Dp = reinterpret_cast<uint16_t*>(ws + L.Dp);
    uint16_t* Dl = reinterpret_cast<uint16_t*>(ws + L.Dl);
    uint16_t* dDl = reinterpret_cast<uint16_t*>(ws + L.dDl);
    uint16_t* dDp = reinterpret_cast<uint16_t*>(ws + L.dDp);
    float* dPm = reinterpret_cast<float*>(ws + L.dPm);
    float* dAm = reinterpret_cast<float*>(ws + L.dAm);

    ChunkArgs fa{a.q, a.k, a.v, a.alpha, a.b, a.w, a.S0, nullptr, nullptr, a.B, a.T, a.H, DK, a.DV,
                 true, ((uint32_t)PRO << 2) | (AS ? 1u : 0u) | (BS ? 2u : 0u), nullptr, 0};
    fa.cu_seqlens = a.cu_seqlens;
    if (!a.saved) {  // recompute the forward's blocks, chunk-start states and D', Delta rows
        const hipError_t e = VAR ? launch_varlen_states(fa, ws, blobs, ring, S_save, Dp, Dl, st)
                                 : launch_split_states(fa, blobs, S_save, Dp, Dl, st);
        if (e != hipSuccess) return e;
    }

    constexpr int DVT = DK < 64 ? DK : 64;
    ChainBwdIO cio{a.v, BS ? a.b : a.w, a.dO, a.dS_T, blobs, G_save, dDl, dDp, a.dv, a.dw, a.dS0};
    cio.dwp = dwp;
    cio.npw = a.DV / 16;
    cio.B = a.B;
    cio.T = a.T;
    cio.H = a.H;
    cio.DV = a.DV;
    cio.nch = nch;
    cio.var = vt;
    cio.ring = ring;
    hipLaunchKernelGGL((bwd_chain_kernel<DK, (PRO & 2) != 0, VAR, BS>), dim3((BH + 7) / 8 * 8 * (a.DV / DVT)),
                       dim3(bwd_chain_threads<DK>()), 0, st, cio);
    // per-chunk kernels: b*h*chunks workgroups, or h * the chunk bound of a packed batch (the ones
    // past the true chunk count leave at once)
    const long items = VAR ? (long)a.H * ring : (long)BH * nch;
    if (items == 0) return hipGetLastError();
    ContractIO xio{a.dO, Dp, Dl, dDl, blobs, dPm, dAm, a.B, a.T, a.H, a.DV, nch};
    xio.var = vt;
    xio.ring = ring;
    hipLaunchKernelGGL((bwd_contract_kernel<DK, VAR>), dim3((unsigned)items), dim3(256), 0, st, xio);
    KeyIO kio{a.q, a.k, a.alpha, a.b, rnq, rnk, a.dO, dDp, Dl, S_save, G_save, dPm, dAm, a.dq, a.dk, a.dalpha, a.db};
    kio.dap = dap;
    kio.dbp = dbp;
    kio.B = a.B;
    kio.T = a.T;
    kio.H = a.H;
    kio.nch = nch;
    kio.var = vt;
    kio.ring = ring;
    hipLaunchKernelGGL((bwd_key_kernel<DK, PRO, VAR, AS, BS>), dim3((unsigned)((items + 7) / 8 * 8 * (DK / 32))),
                       dim3(256), 0, st, kio);
    if constexpr ((PRO & 1) != 0) {  // dq, dk through the L2 norm
        const long rows = (VAR ? 1l : (long)a.B) * a.T * a.H;
        constexpr int RPB = 256 / (DK / 4);
        const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
        hipLaunchKernelGGL(l2norm_bwd<DK>, grid, dim3(256), 0, st, a.dq, static_cast<const uint16_t*>(a.q), rnq, rows);
        hipLaunchKernelGGL(l2norm_bwd<DK>, grid, dim3(256), 0, st, a.dk, static_cast<const uint16_t*>(a.k), rnk, rows);
    }
    return hipGetLastError();
}

}  // namespace

// Extra workspace for scalar gates: the per-row partial sums of their gradients (fp32: DK / 32
// per row for alpha and for b, DV / 16 for the w side of a scalar beta); for the L2 norm: the
// reciprocal row norms of q and k.
struct ScalarLayout {
    size_t dap, dbp, dwp, rnq, rnk, total;
};

ScalarLayout scalar_layout(size_t base, size_t rows, int DK, int DV, uint32_t flags) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const bool as = (flags & 1u) != 0, bs = (flags & 2u) != 0;
    ScalarLayout L{};
    size_t o = base;
    L.dap = o;
    o += as ? up(rows * (DK / 32) * 4) : 0;
    L.dbp = o;
    o += bs ? up(rows * (DK / 32) * 4) : 0;
    L.dwp = o;
    o += bs ? up(rows * (DV / 16) * 4) : 0;
    const bool l2n = (flags & 4u) != 0;  // the row norms of q and k
    L.rnq = o;
    o += l2n ? up(rows * 4) : 0;
    L.rnk = o;
    o += l2n ? up(rows * 4) : 0;
    L.total = o;
    return L;
}

bool bwd_supported(int T, int H, int DK, int DV, bool bf16, uint32_t flags) {
    if (!bf16 || (flags & ~15u) != 0u || DK != DV) return false;
    if (DK != 32 && DK != 64 && DK != 128) return false;
    // one sequence's rows, the last chunk's rows past T included, addressed with 32-bit offsets
    return ((long long)T + CH) * H * DV * 4 < (1ll << 32);
}

size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV, uint32_t flags) {
    const size_t base = bwd_layout(B, T, H, DK, DV).total;
    return (flags & 7u) ? scalar_layout(base, (size_t)B * T * H, DK, DV, flags).total : base;
}

size_t bwd_varlen_workspace_bytes(int n, int T, int H, int DK, int DV, uint32_t flags) {
    const size_t base = bwd_layout_var(n, T, H, DK, DV).total;
    return (flags & 7u) ? scalar_layout(base, (size_t)T * H, DK, DV, flags).total : base;
}

hipError_t launch_fwd_save(const ChunkArgs& a, hipStream_t s) {
    if (!a.bf16 || !bwd_supported(a.T, a.H, a.DK, a.DV, true, a.flags)) return hipErrorNotSupported;
    if (a.T == 0) return hipSuccess;
    const bool var = a.cu_seqlens != nullptr;  // packed batch: a.B sequences, a.T rows in all
    const size_t need = var ? bwd_varlen_workspace_bytes(a.B, a.T, a.H, a.DK, a.DV, a.flags)
                            : bwd_workspace_bytes(a.B, a.T, a.H, a.DK, a.DV, a.flags);
    if (!a.workspace || a.workspace_bytes < need) return hipErrorInvalidValue;
    // the places launch_bwd reads them from: the blocks, the saves and (packed) the sequence
    // table at the start of the workspace
    const BwdLayout L = var ? bwd_layout_var(a.B, a.T, a.H, a.DK, a.DV) : bwd_layout(a.B, a.T, a.H, a.DK, a.DV);
    char* ws = static_cast<char*>(a.workspace);
    uint16_t* S_save = reinterpret_cast<uint16_t*>(ws + L.S_save);
    uint16_t* Dp = reinterpret_cast<uint16_t*>(ws + L.Dp);
    uint16_t* Dl = reinterpret_cast<uint16_t*>(ws + L.Dl);
    return var ? launch_varlen_states(a, ws, ws + L.blobs, varlen_chunk_bound(a.B, a.T), S_save, Dp, Dl, s)
               : launch_split_states(a, ws + L.blobs, S_save, Dp, Dl, s);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
    if (!bwd_supported(a.T, a.H, a.DK, a.DV, a.bf16, a.flags)) return hipErrorNotSupported;
    if (a.T == 0) {  // no tokens: dS0 = dS_T (or zeros), nothing else to write
        if (!a.dS0) return hipSuccess;
        const long n = (long)a.B * a.H * a.DK * a.DV;
        hipLaunchKernelGGL(copy_or_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.dS0, a.dS_T, n);
        return hipGetLastError();
    }
    const bool var = a.cu_seqlens != nullptr;  // packed batch: a.B sequences, a.T rows in all
    const size_t need = var ? bwd_varlen_workspace_bytes(a.B, a.T, a.H, a.DK, a.DV, a.flags)
                            : bwd_workspace_bytes(a.B, a.T, a.H, a.DK, a.DV, a.flags);
    if (!a.workspace || a.workspace_bytes < need) return hipErrorInvalidValue;
    const BwdArgs& g = a;
    const bool as = (a.flags & 1u) != 0, bs = (a.flags & 2u) != 0, l2n = (a.flags & 4u) != 0;
    const long rows = (var ? 1l : (long)a.B) * a.T * a.H;  // token rows
    const size_t base = var ? bwd_layout_var(a.B, a.T, a.H, a.DK, a.DV).total : bwd_layout(a.B, a.T, a.H, a.DK, a.DV).total;
    const ScalarLayout L = scalar_layout(base, (size_t)rows, a.DK, a.DV, a.flags);
    char* ws = static_cast<char*>(a.workspace);
    float* rnq = nullptr;
    float* rnk = nullptr;
    if (l2n) {  // the reciprocal row norms of q and k, as the forward takes them
        rnq = reinterpret_cast<float*>(ws + L.rnq);
        rnk = reinterpret_cast<float*>(ws + L.rnk);
        auto norms = [&](auto dk) {
            constexpr int D = decltype(dk)::value, RPB = 256 / (D / 8);
            const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
            hipLaunchKernelGGL(row_rnorm<D>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(a.q), rnq, rows);
            hipLaunchKernelGGL(row_rnorm<D>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(a.k), rnk, rows);
        };
        if (a.DK == 32) norms(std::integral_constant<int, 32>());
        else if (a.DK == 64) norms(std::integral_constant<int, 64>());
        else norms(std::integral_constant<int, 128>());
    }
    float* dap = as ? reinterpret_cast<float*>(ws + L.dap) : nullptr;
    float* dbp = bs ? reinterpret_cast<float*>(ws + L.dbp) : nullptr;
    float* dwp = bs ? reinterpret_cast<float*>(ws + L.dwp) : nullptr;
    auto gates = [&](auto dk, auto pro, auto vr) -> hipError_t {
        constexpr int D = decltype(dk)::value, PRO = decltype(pro)::value;
        constexpr bool V = decltype(vr)::value;
        switch (a.flags & 3u) {
            case 0: return launch_bwd_t<D, PRO, V, false, false>(g, rnq, rnk, dap, dbp, dwp, s);
            case 1: return launch_bwd_t<D, PRO, V, true, false>(g, rnq, rnk, dap, dbp, dwp, s);
            case 2: return launch_bwd_t<D, PRO, V, false, true>(g, rnq, rnk, dap, dbp, dwp, s);
            default: return launch_bwd_t<D, PRO, V, true, true>(g, rnq, rnk, dap, dbp, dwp, s);
        }
    };
    auto go = [&](auto pro) -> hipError_t {
        auto with = [&](auto vr) -> hipError_t {
            switch (a.DK) {
                case 32: return gates(std::integral_constant<int, 32>(), pro, vr);
                case 64: return gates(std::integral_constant<int, 64>(), pro, vr);
                case 128: return gates(std::integral_constant<int, 128>(), pro, vr);
                default: return hipErrorNotSupported;
            }
        };
        return var ? with(std::true_type()) : with(std::false_type());
    };
    hipError_t e;
    switch ((a.flags >> 2) & 3u) {
        case 0: e = go(std::integral_constant<int, 0>()); break;
        case 1: e = go(std::integral_constant<int, 1>()); break;
        case 2: e = go(std::integral_constant<int, 2>()); break;
        default: e = go(std::integral_constant<int, 3>()); break;
    }
    if (e != hipSuccess || !(as || bs)) return e;
    hipLaunchKernelGGL(scalar_gate_sums, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, dap, a.DK / 32, dbp,
                       a.DK / 32, dwp, a.DV / 16, a.dalpha, a.db, rows);
    return hipGetLastError();
}

}  // namespace gdn2
