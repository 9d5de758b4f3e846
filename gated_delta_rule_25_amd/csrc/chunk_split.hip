// chunk_split.hip -- host side of the two-kernel prefill (prep_kernel, chain_kernel) for
// batches of equal-length sequences: the ring of chunk ranges, and segments for long sequences
// with few (b, h).
#include "chunk_split_kernels.h"

namespace gdn2 {

namespace {

using namespace chunk;


// Value columns per chain workgroup: 64, or d below that.
constexpr int split_dvt(int DK) { return DK < 64 ? DK : 64; }

// Segments for a long sequence with few (b, h): enough that the chain fills the chip, each at
// least 16 chunks long. nseg = 1 means no segmentation.
struct SplitPlan {
    int nseg, seg_len;
    size_t extra_bytes;  // Psi/Phi and the segment start states
};

SplitPlan split_plan(int B, int T, int H, int DK, int DV) {
    const int nch = (T + CH - 1) / CH;
    const int DVT = split_dvt(DK);
    const long wgs = (long)B * H * (DV / DVT);
    SplitPlan p{1, nch, 0};
    if (wgs < 256 && nch >= 32) {
        int g = (int)((256 + wgs - 1) / wgs);
        if (g > nch / 16) g = nch / 16;
        if (g >= 2) {
            p.seg_len = (nch + g - 1) / g;
            p.nseg = (nch + p.seg_len - 1) / p.seg_len;
            const size_t BH = (size_t)B * H;
            p.extra_bytes = (BH * (p.nseg - 1) * DK * (DV + DK) + BH * p.nseg * DK * DV) * 4;
        }
    }
    return p;
}

template <int DK, bool BF16, bool AS, bool BS, int PRO>
hipError_t launch_split_t(const ChunkArgs& a, hipStream_t st) {
    constexpr bool WS = (PRO & 2) != 0 && !BS;  // w through the sigmoid in the chain
    constexpr int DVT = split_dvt(DK);
    using BL = Blob<DK, BF16>;
    const int BH = a.B * a.H, BHp = (BH + 7) / 8 * 8;
    const int nch = (a.T + CH - 1) / CH;
    const size_t state_bytes = (size_t)BH * a.DK * a.DV * 4;
    float* Sbuf = a.S_out;
    char* ws = static_cast<char*>(a.workspace);
    if (!Sbuf) {
        Sbuf = reinterpret_cast<float*>(ws);
        ws += state_bytes;
    }
    const size_t avail = a.workspace_bytes - (a.S_out ? 0 : state_bytes);
    const size_t per_chunk = (size_t)BH * BL::bytes;
    const int tiles = a.DV / DVT;
    const SplitPlan plan = split_plan(a.B, a.T, a.H, DK, a.DV);
    const long ld = DK;  // state rows are DK long in k, DV in v
    if (plan.nseg > 1 && avail >= (size_t)nch * per_chunk + plan.extra_bytes) {
        // segments: prep over all chunks; each segment's transition (Psi, Phi) from the state
        // recurrence alone; a scan for every segment's start state; then all segments at once
        const int G = plan.nseg;
        float* psiphi = reinterpret_cast<float*>(ws + (size_t)nch * per_chunk);
        float* sseg = psiphi + (size_t)BH * (G - 1) * DK * (a.DV + DK);
        hipLaunchKernelGGL((prep_kernel<DK, BF16, AS, BS, PRO>), dim3(BH * nch), dim3(256), 0, st, a.q, a.k, a.alpha,
                           a.b, a.B, a.T, a.H, 0, nch, ws, VarTab{});
        const ChainIO tr{a.v, a.w, a.o, ws, nch, 0, nch, plan.seg_len, G - 1, a.B, a.T, a.H, a.DV,
                         nullptr, 0, 0, a.DV,
                         psiphi, (long)(G - 1) * DK * (a.DV + DK), ld * (a.DV + DK), a.DV + DK, 0};
        ChainIO trp = tr;
        trp.phi_tiles = DK / DVT;
        hipLaunchKernelGGL((chain_kernel<DK, DVT, BF16, BS, true, false, WS>), dim3((G - 1) * BHp * (tiles + DK / DVT)),
                           dim3(ChainSmem<DK, DVT, BF16, true>::threads), 0, st, trp);
        hipLaunchKernelGGL((scan_kernel<DK>), dim3(BH * (a.DV / 8)), dim3(256), 0, st, a.S0, psiphi, sseg, G, a.DV);
        const ChainIO fu{a.v, a.w, a.o, ws, nch, 0, nch, plan.seg_len, G, a.B, a.T, a.H, a.DV,
                         sseg, (long)G * DK * a.DV, ld * a.DV, a.DV,
                         Sbuf, ld * a.DV, 0, a.DV, 1};
        hipLaunchKernelGGL((chain_kernel<DK, DVT, BF16, BS, false, false, WS>), dim3(G * BHp * tiles), dim3(ChainSmem<DK, DVT, BF16>::threads), 0,
                           st, fu);
        return hipGetLastError();
    }
    int R = (int)(avail / per_chunk);
    if (R < 1) return hipErrorInvalidValue;
    if (R > nch) R = nch;
    for (int n0 = 0; n0 < nch; n0 += R) {
        const int cnt = nch - n0 < R ? nch - n0 : R;
        hipLaunchKernelGGL((prep_kernel<DK, BF16, AS, BS, PRO>), dim3(BH * cnt), dim3(256), 0, st, a.q, a.k,
                           a.alpha, a.b, a.B, a.T, a.H, n0, cnt, ws, VarTab{});
        const ChainIO io{a.v, a.w, a.o, ws, cnt, n0, n0 + cnt, cnt, 1, a.B, a.T, a.H, a.DV,
                         n0 == 0 ? a.S0 : Sbuf, ld * a.DV, 0, a.DV,
                         Sbuf, ld * a.DV, 0, a.DV, 0};
        hipLaunchKernelGGL((chain_kernel<DK, DVT, BF16, BS, false, false, WS>), dim3(BHp * tiles), dim3(ChainSmem<DK, DVT, BF16>::threads), 0, st,
                           io);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, bool BF16, int PRO>
hipError_t launch_split_gates(const ChunkArgs& a, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_split_t<DK, BF16, false, false, PRO>(a, s);
        case 1: return launch_split_t<DK, BF16, true, false, PRO>(a, s);
        case 2: return launch_split_t<DK, BF16, false, true, PRO>(a, s);
        default: return launch_split_t<DK, BF16, true, true, PRO>(a, s);
    }
}

template <int DK, bool BF16>
hipError_t launch_split_flags(const ChunkArgs& a, hipStream_t s) {
    switch ((a.flags >> 2) & 3u) {  // prologue: L2 norm of q, k (1), gate pre-activations (2)
        case 0: return launch_split_gates<DK, BF16, 0>(a, s);
        case 1: return launch_split_gates<DK, BF16, 1>(a, s);
        case 2: return launch_split_gates<DK, BF16, 2>(a, s);
        default: return launch_split_gates<DK, BF16, 3>(a, s);
    }
}

template <int DK, int PRO, bool AS, bool BS>
hipError_t launch_states_t(const ChunkArgs& a, char* blobs, uint16_t* S_save, uint16_t* Dp_save, uint16_t* Dl_save,
                           hipStream_t st) {
    constexpr int DVT = split_dvt(DK);
    const int BH = a.B * a.H, BHp = (BH + 7) / 8 * 8;
    const int nch = (a.T + CH - 1) / CH;
    hipLaunchKernelGGL((prep_kernel<DK, true, AS, BS, PRO>), dim3(BH * nch), dim3(256), 0, st, a.q, a.k,
                       a.alpha, a.b, a.B, a.T, a.H, 0, nch, blobs, VarTab{});
    // with a.o: the forward itself (o and S_T) with the saves; without: the saves alone
    ChainIO io{a.v, a.w, a.o, blobs, nch, 0, nch, nch, 1, a.B, a.T, a.H, a.DV,
               a.S0, (long)DK * a.DV, 0, a.DV, a.o ? a.S_out : nullptr, (long)DK * a.DV, 0, a.DV, 0};
    io.S_save = S_save;
    io.save_nch = nch;
    io.Dp_save = Dp_save;
    io.Dl_save = Dl_save;
    if (a.o)
        hipLaunchKernelGGL((chain_kernel<DK, DVT, true, BS, false, true, (PRO & 2) != 0>), dim3(BHp * (a.DV / DVT)),
                           dim3(ChainSmem<DK, DVT, true>::threads), 0, st, io);
    else
        hipLaunchKernelGGL((chain_kernel<DK, DVT, true, BS, true, true, (PRO & 2) != 0>), dim3(BHp * (a.DV / DVT)),
                           dim3(ChainSmem<DK, DVT, true>::threads), 0, st, io);
    return hipGetLastError();
}

template <int DK, int PRO>
hipError_t launch_states_gates(const ChunkArgs& a, char* blobs, uint16_t* S_save, uint16_t* Dp_save,
                               uint16_t* Dl_save, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_states_t<DK, PRO, false, false>(a, blobs, S_save, Dp_save, Dl_save, s);
        case 1: return launch_states_t<DK, PRO, true, false>(a, blobs, S_save, Dp_save, Dl_save, s);
        case 2: return launch_states_t<DK, PRO, false, true>(a, blobs, S_save, Dp_save, Dl_save, s);
        default: return launch_states_t<DK, PRO, true, true>(a, blobs, S_save, Dp_save, Dl_save, s);
    }
}

}  // namespace

hipError_t launch_split_states(const ChunkArgs& a, char* blobs, uint16_t* S_save, uint16_t* Dp_save, uint16_t* Dl_save,
                               hipStream_t s) {
    if (!a.bf16 || (a.flags & ~15u) != 0u || !split_supported(a.T, a.H, a.DK, a.DV, true)) return hipErrorNotSupported;
    auto go = [&](auto pro) -> hipError_t {
        constexpr int PRO = decltype(pro)::value;
        switch (a.DK) {
            case 32: return launch_states_gates<32, PRO>(a, blobs, S_save, Dp_save, Dl_save, s);
            case 64: return launch_states_gates<64, PRO>(a, blobs, S_save, Dp_save, Dl_save, s);
            case 128: return launch_states_gates<128, PRO>(a, blobs, S_save, Dp_save, Dl_save, s);
            default: return hipErrorNotSupported;
        }
    };
    switch ((a.flags >> 2) & 3u) {  // prologue flags, as the forward takes them
        case 0: return go(std::integral_constant<int, 0>());
        case 1: return go(std::integral_constant<int, 1>());
        case 2: return go(std::integral_constant<int, 2>());
        default: return go(std::integral_constant<int, 3>());
    }
}

bool split_supported(int T, int H, int DK, int DV, bool bf16) {
    if (DK != DV || T < 0) return false;
    if (bf16) return DK == 32 || DK == 64 || DK == 128;
    return DK == 32;  // packed batches take fp32 blocks of d = 32 only
}

// gdn2_chunk_fwd's equal-length batches also take bf16 at d = 256 and fp32 at d = 64 and 128 (one
// block buffer in the chain kernel); the packed batches and the backward's state pass stay at
// the sizes above.
bool split_fwd_supported(int T, int H, int DK, int DV, bool bf16) {
    if (split_supported(T, H, DK, DV, bf16)) return true;
    if (DK != DV || T < 0) return false;
    return bf16 ? DK == 256 : (DK == 64 || DK == 128);
}

size_t split_workspace_bytes(int B, int T, int H, int DK, int DV, bool bf16) {
    const size_t nch = ((size_t)T + CH - 1) / CH;
    const SplitPlan plan = split_plan(B, T, H, DK, DV);
    return (size_t)B * H * DK * DV * 4 + nch * split_chunk_bytes(B, H, DK, bf16) + plan.extra_bytes;
}

size_t split_chunk_bytes(int B, int H, int DK, bool bf16) {
    size_t blob = 0;
    if (bf16) {
        blob = DK == 32    ? Blob<32, true>::bytes
               : DK == 64  ? Blob<64, true>::bytes
               : DK == 128 ? Blob<128, true>::bytes
                           : Blob<256, true>::bytes;
    } else {
        blob = DK == 32 ? Blob<32, false>::bytes : DK == 64 ? Blob<64, false>::bytes : Blob<128, false>::bytes;
    }
    return (size_t)B * H * blob;
}

hipError_t launch_split(const ChunkArgs& a, hipStream_t s) {
    if (!split_fwd_supported(a.T, a.H, a.DK, a.DV, a.bf16)) return hipErrorNotSupported;
    if (a.bf16) {
        switch (a.DK) {
            case 32: return launch_split_flags<32, true>(a, s);
            case 64: return launch_split_flags<64, true>(a, s);
            case 128: return launch_split_flags<128, true>(a, s);
            case 256: return launch_split_flags<256, true>(a, s);
            default: return hipErrorNotSupported;
        }
    }
    switch (a.DK) {
        case 32: return launch_split_flags<32, false>(a, s);
        case 64: return launch_split_flags<64, false>(a, s);
        case 128: return launch_split_flags<128, false>(a, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace gdn2
