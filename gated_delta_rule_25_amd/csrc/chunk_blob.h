// chunk_blob.h -- the per-chunk operand block of the two-kernel prefill (written by the prep
// kernel, read by the forward and backward chain kernels) and the LDS copy helpers around it.
#pragma once

#include "chunk_common.h"

namespace gdn2 {
namespace chunk {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// Per-chunk operand blob (also the chain kernel's LDS buffer layout). Matrices are addressed
// through en() (E_hat, Q_hat: [64][DK]), kbt() (K_bar^T: [DK][64]) and tp() (T, P: [64][64],
// lower block triangular), in elements; the chain kernel reads 4-element units of 16 consecutive
// rows at one column, and the layouts give those 16 reads distinct LDS banks.
//  - fp16: no padding. Within a row the 4-element (8-byte) units are permuted by an XOR with the
//    row index (row & 15 for rows of 64 dwords or more; (row >> 1) & 7 for rows of 16 dwords,
//    whose consecutive rows already alternate between the two halves of the banks). T and P keep
//    only the column blocks the chain reads: 32 columns for rows 0..31, 64 for rows 32..63.
//  - fp32: rows padded by 4 elements, full 64x64 T and P.
template <int DK, bool F16>
struct Blob {
    using E = typename Prec<F16>::E;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int PAD = F16 ? 0 : 4;
    static constexpr int DKP = DK + PAD, CHP = CH + PAD;
    static constexpr int TPE = F16 ? 32 * 32 + 32 * 64 : CH * CHP;  // elements of T or P
    __device__ static int unit_sw(int r, int width) { return width >= 64 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static int sw(int r, int c, int width) {
        return F16 ? ((((c >> 2) ^ unit_sw(r, width)) << 2) | (c & 3)) : c;
    }
    __device__ static int en(int r, int c) { return r * DKP + sw(r, c, DK); }
    __device__ static int kbt(int r, int c) { return r * CHP + sw(r, c, CH); }
    __device__ static int tp(int r, int c) {
        if constexpr (F16) return r < 32 ? r * 32 + sw(r, c, 32) : 32 * 32 + (r - 32) * 64 + sw(r, c, 64);
        return r * CHP + c;
    }
    // The state recurrence alone needs the prefix [En .. beta]; the outputs also need P and Q_hat.
    static constexpr int oEn = 0;                       // E_hat, negated
    static constexpr int oKbT = oEn + CH * DKP * ES;    // K_bar^T
    static constexpr int oTm = oKbT + DK * CHP * ES;    // T
    static constexpr int oGC = oTm + TPE * ES;          // float [DK]    gamma_last
    static constexpr int oBeta = oGC + DK * 4;          // float [64]    scalar beta per row (scalar-beta gates)
    static constexpr int stateBytes = oBeta + CH * 4;
    static constexpr int oP = stateBytes;               // P
    static constexpr int oQh = oP + TPE * ES;           // Q_hat
    static constexpr int bytes = (oQh + CH * DKP * ES + 255) / 256 * 256;
    static_assert(stateBytes % 16 == 0 && oP % 16 == 0, "16-byte copies");
};

// Copy `bytes` (a multiple of 16) from global to LDS with `nw` wavefronts (this one is `cw`),
// 1 KiB per instruction: lane i moves 16 bytes to LDS base + 16 i. Counted by vmcnt; the
// caller waits.
__device__ __forceinline__ void dma_flat(const char* g, char* l, int bytes, int cw, int nw, int lane) {
    for (int off = cw * 1024; off < bytes; off += nw * 1024) {
        if (off + lane * 16 < bytes)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(g + off + lane * 16), (lds_ptr_t)(l + off), 16, 0, 0);
    }
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// All but the newest N (< 64) vector-memory operations done (vmcnt(N): low 4 bits in [3:0],
// high 2 bits in [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_but() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Packed (ragged) batch: sequence s holds token rows [start[s], start[s] + len[s]) of the packed
// inputs and chunks [coff[s], coff[s + 1]) of the batch; n sequences. Built on the device from
// the caller's cumulative sequence lengths.
struct VarTab {
    const int* coff = nullptr;
    const int* start = nullptr;
    const int* len = nullptr;
    const int* perm = nullptr;  // the sequences, longest first (the chains' dispatch order)
    int n = 0;
};

// The sequence that holds chunk gc of a packed batch: the last s with coff[s] <= gc (gc below the
// chunk count, so that sequence has a chunk at gc - coff[s]).
__device__ __forceinline__ int varlen_seq_of(const VarTab& vt, int gc) {
    int lo = 0, hi = vt.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (vt.coff[mid] <= gc) {
            lo = mid;
        } else {
            hi = mid - 1;
        }
    }
    return lo;
}

}  // namespace chunk
}  // namespace gdn2
