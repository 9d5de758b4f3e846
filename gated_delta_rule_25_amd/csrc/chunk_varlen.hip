// chunk_varlen.hip -- the two-kernel prefill (prep_kernel, chain_kernel) over a packed batch of
// sequences of different lengths.
//
// The sequences lie back to back along the token axis ([T_total, H, d] rows) and are delimited
// by cumulative lengths cu[0..n] that live on the device. Each sequence is chunked from its own
// first token [page "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph
// "Реализация": the chunkwise form restarts from the sequence's initial state], so a chunk never
// spans two sequences. The host never reads cu: a one-workgroup kernel turns it into the
// sequence table (first row, length, first chunk), prep runs over an upper bound of the chunk
// count (the workgroups past the true count leave at once), and the chain runs one workgroup per
// (sequence, head, value tile).
#include "chunk_split_kernels.h"

namespace gdn2 {

namespace {

using namespace chunk;

// Sequence table from cu[0..n]: each bound is clamped to [0, T] and the bounds are made
// non-decreasing (a running maximum), so any input gives sequences that partition rows inside
// the batch; start[s] = cu'[s], len[s] = cu'[s+1] - cu'[s], and coff[s] = the sum of
// ceil(len / C) over the sequences before s (coff[n] = the chunk count). One workgroup walks the
// bounds in tiles of 256 with two block scans per tile. Then perm[0..n) lists the sequences by
// decreasing chunk count (a counting sort over min(chunks, kBuckets - 1); the order inside a
// bucket is whatever the atomics give, which changes no result: the chains of different
// sequences share nothing).
constexpr int kBuckets = 1024;

__global__ void __launch_bounds__(256) varlen_table_kernel(const int* __restrict__ cu, int n, int T,
                                                           int* __restrict__ coff, int* __restrict__ start,
                                                           int* __restrict__ len, int* __restrict__ perm) {
    __shared__ int smax[256], ssum[256], tail[2];
    __shared__ int hist[kBuckets];
    const int tid = threadIdx.x;
    int cmax = 0, csum = 0;  // running maximum and chunk sum carried from the previous tiles
    for (int base = 0; base <= n; base += 256) {
        const int i = base + tid;
        smax[tid] = i <= n ? min(max(cu[i], 0), T) : 0;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {  // inclusive max scan (all values are >= 0)
            const int y = tid >= d ? smax[tid - d] : 0;
            __syncthreads();
            smax[tid] = max(smax[tid], y);
            __syncthreads();
        }
        const int M = max(smax[tid], cmax);
        const int Mp = tid > 0 ? max(smax[tid - 1], cmax) : cmax;  // bound i - 1
        const int l = M - Mp;
        ssum[tid] = (i >= 1 && i <= n) ? (l + CH - 1) / CH : 0;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {  // inclusive sum scan of the chunk counts
            const int y = tid >= d ? ssum[tid - d] : 0;
            __syncthreads();
            ssum[tid] += y;
            __syncthreads();
        }
        const int S = ssum[tid] + csum;
        if (i <= n) coff[i] = S;
        if (i < n) start[i] = M;
        if (i >= 1 && i <= n) len[i - 1] = l;
        if (tid == 255) {
            tail[0] = M;
            tail[1] = S;
        }
        __syncthreads();
        cmax = tail[0];
        csum = tail[1];
        __syncthreads();  // tail and the scan arrays are rewritten by the next tile
    }
    // bucket b = kBuckets - 1 - min(chunks, kBuckets - 1): bucket 0 holds the longest sequences
    for (int i = tid; i < kBuckets; i += 256) hist[i] = 0;
    __syncthreads();  // (also orders this workgroup's writes of len above before the reads below)
    auto bucket = [&](int s) {
        const int c = (len[s] + CH - 1) / CH;
        return kBuckets - 1 - (c < kBuckets - 1 ? c : kBuckets - 1);
    };
    for (int s = tid; s < n; s += 256) atomicAdd(&hist[bucket(s)], 1);
    __syncthreads();
    // exclusive scan of the kBuckets counts: 4 per thread, then one block scan of the sums
    constexpr int PER = kBuckets / 256;
    int loc[PER], acc = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        loc[e] = acc;
        acc += hist[tid * PER + e];
    }
    ssum[tid] = acc;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {  // inclusive sum scan
        const int y = tid >= d ? ssum[tid - d] : 0;
        __syncthreads();
        ssum[tid] += y;
        __syncthreads();
    }
    const int before = ssum[tid] - acc;  // the counts of the buckets below this thread's
#pragma unroll
    for (int e = 0; e < PER; ++e) hist[tid * PER + e] = before + loc[e];
    __syncthreads();
    for (int s = tid; s < n; s += 256) perm[atomicAdd(&hist[bucket(s)], 1)] = s;
}

template <int DK, bool BF16, bool AS, bool BS, int PRO>
hipError_t launch_varlen_t(const ChunkArgs& a, hipStream_t st) {
    constexpr bool WS = (PRO & 2) != 0 && !BS;  // w through the sigmoid in the chain
    constexpr int DVT = DK < 64 ? DK : 64;
    const int N = a.B;
    const long ring = varlen_chunk_bound(N, a.T);
    char* ws = static_cast<char*>(a.workspace);
    int* coff = reinterpret_cast<int*>(ws);
    int* start = coff + N + 1;
    int* len = start + N;
    int* perm = len + N;
    char* blobs = ws + varlen_table_bytes(N);
    VarTab vt;
    vt.coff = coff;
    vt.start = start;
    vt.len = len;
    vt.perm = perm;
    vt.n = N;
    hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, N, a.T, coff, start, len, perm);
    if (ring > 0)
        hipLaunchKernelGGL((prep_kernel<DK, BF16, AS, BS, PRO, true>), dim3((unsigned)(a.H * ring)), dim3(256), 0, st,
                           a.q, a.k, a.alpha, a.b, 1, a.T, a.H, 0, (int)ring, blobs, vt);
    const long ld = DK;
    ChainIO io{a.v, a.w, a.o, blobs, (int)ring, 0, 0, 0, 1, N, a.T, a.H, a.DV,
               a.S0, ld * a.DV, 0, a.DV,
               a.S_out, ld * a.DV, 0, a.DV, 0};
    io.var = vt;
    const int BH = N * a.H, BHp = (BH + 7) / 8 * 8;
    hipLaunchKernelGGL((chain_kernel<DK, DVT, BF16, BS, false, false, WS, true>), dim3(BHp * (a.DV / DVT)),
                       dim3(ChainSmem<DK, DVT, BF16>::threads), 0, st, io);
    return hipGetLastError();
}

// The backward's forward pass over a packed batch: the sequence table (at `table`), prep into
// `blobs` ([h][chunk of the batch], `ring` slots per head) and the chain with saves (state-only,
// or with o and S_T when a.o is set):
// the start state of every chunk ([h][chunk of the batch][DK][DV]) and the rows of D' and Delta
// (fp16, packed rows). bf16, scalar gate forms AS / BS, the prologue flags PRO.
template <int DK, int PRO, bool AS, bool BS>
hipError_t launch_varlen_states_t(const ChunkArgs& a, char* table, char* blobs, long ring, uint16_t* S_save,
                                  uint16_t* Dp_save, uint16_t* Dl_save, hipStream_t st) {
    constexpr int DVT = DK < 64 ? DK : 64;
    const int N = a.B;
    VarTab vt;
    vt.coff = reinterpret_cast<int*>(table);
    vt.start = vt.coff + N + 1;
    vt.len = vt.start + N;
    vt.perm = vt.len + N;
    vt.n = N;
    hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, N, a.T, const_cast<int*>(vt.coff),
                       const_cast<int*>(vt.start), const_cast<int*>(vt.len), const_cast<int*>(vt.perm));
    if (ring > 0)
        hipLaunchKernelGGL((prep_kernel<DK, true, AS, BS, PRO, true>), dim3((unsigned)(a.H * ring)), dim3(256), 0,
                           st, a.q, a.k, a.alpha, a.b, 1, a.T, a.H, 0, (int)ring, blobs, vt);
    const long ld = DK;
    // with a.o: the forward itself (o and S_T) with the saves; without: the saves alone
    ChainIO io{a.v, a.w, a.o, blobs, (int)ring, 0, 0, 0, 1, N, a.T, a.H, a.DV,
               a.S0, ld * a.DV, 0, a.DV, a.o ? a.S_out : nullptr, ld * a.DV, 0, a.DV, 0};
    io.var = vt;
    io.S_save = S_save;
    io.Dp_save = Dp_save;
    io.Dl_save = Dl_save;
    const int BH = N * a.H, BHp = (BH + 7) / 8 * 8;
    if (a.o)
        hipLaunchKernelGGL((chain_kernel<DK, DVT, true, BS, false, true, (PRO & 2) != 0, true>),
                           dim3(BHp * (a.DV / DVT)), dim3(ChainSmem<DK, DVT, true>::threads), 0, st, io);
    else
        hipLaunchKernelGGL((chain_kernel<DK, DVT, true, BS, true, true, (PRO & 2) != 0, true>),
                           dim3(BHp * (a.DV / DVT)), dim3(ChainSmem<DK, DVT, true>::threads), 0, st, io);
    return hipGetLastError();
}

template <int DK, int PRO>
hipError_t launch_varlen_states_gates(const ChunkArgs& a, char* table, char* blobs, long ring, uint16_t* S_save,
                                      uint16_t* Dp_save, uint16_t* Dl_save, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_varlen_states_t<DK, PRO, false, false>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
        case 1: return launch_varlen_states_t<DK, PRO, true, false>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
        case 2: return launch_varlen_states_t<DK, PRO, false, true>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
        default: return launch_varlen_states_t<DK, PRO, true, true>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
    }
}

template <int DK, bool BF16, int PRO>
hipError_t launch_varlen_gates(const ChunkArgs& a, hipStream_t s) {
    switch (a.flags & 3u) {
        case 0: return launch_varlen_t<DK, BF16, false, false, PRO>(a, s);
        case 1: return launch_varlen_t<DK, BF16, true, false, PRO>(a, s);
        case 2: return launch_varlen_t<DK, BF16, false, true, PRO>(a, s);
        default: return launch_varlen_t<DK, BF16, true, true, PRO>(a, s);
    }
}

template <int DK, bool BF16>
hipError_t launch_varlen_flags(const ChunkArgs& a, hipStream_t s) {
    switch ((a.flags >> 2) & 3u) {
        case 0: return launch_varlen_gates<DK, BF16, 0>(a, s);
        case 1: return launch_varlen_gates<DK, BF16, 1>(a, s);
        case 2: return launch_varlen_gates<DK, BF16, 2>(a, s);
        default: return launch_varlen_gates<DK, BF16, 3>(a, s);
    }
}

}  // namespace

long varlen_chunk_bound(int n, int T) {
    // sum over sequences of ceil(len / C) <= (sum of len + (C - 1) n) / C
    return ((long)T + (long)(CH - 1) * n) / CH;
}

size_t varlen_table_bytes(int n) { return ((size_t)(4 * (size_t)n + 1) * 4 + 255) / 256 * 256; }

size_t varlen_workspace_bytes(int n, int T, int H, int DK, int DV, bool bf16) {
    return varlen_table_bytes(n) + (size_t)varlen_chunk_bound(n, T) * split_chunk_bytes(1, H, DK, bf16);
}

hipError_t launch_varlen_states(const ChunkArgs& a, char* table, char* blobs, long ring, uint16_t* S_save,
                                uint16_t* Dp_save, uint16_t* Dl_save, hipStream_t s) {
    if (!a.bf16 || (a.flags & ~15u) != 0u || !a.cu_seqlens || !split_supported(a.T, a.H, a.DK, a.DV, true))
        return hipErrorNotSupported;
    auto go = [&](auto pro) -> hipError_t {
        constexpr int PRO = decltype(pro)::value;
        switch (a.DK) {
            case 32: return launch_varlen_states_gates<32, PRO>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
            case 64: return launch_varlen_states_gates<64, PRO>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
            case 128: return launch_varlen_states_gates<128, PRO>(a, table, blobs, ring, S_save, Dp_save, Dl_save, s);
            default: return hipErrorNotSupported;
        }
    };
    switch ((a.flags >> 2) & 3u) {
        case 0: return go(std::integral_constant<int, 0>());
        case 1: return go(std::integral_constant<int, 1>());
        case 2: return go(std::integral_constant<int, 2>());
        default: return go(std::integral_constant<int, 3>());
    }
}

// The packed forward takes the sizes of the equal-length two-kernel path except head size 256:
// bf16 and fp32 at d in {32, 64, 128}.
bool varlen_fwd_supported(int T, int H, int DK, int DV, bool bf16) {
    return DK == DV && T >= 0 && (DK == 32 || DK == 64 || DK == 128);
}

hipError_t launch_split_varlen(const ChunkArgs& a, hipStream_t s) {
    if (!varlen_fwd_supported(a.T, a.H, a.DK, a.DV, a.bf16) || !a.cu_seqlens) return hipErrorNotSupported;
    if (a.bf16) {
        switch (a.DK) {
            case 32: return launch_varlen_flags<32, true>(a, s);
            case 64: return launch_varlen_flags<64, true>(a, s);
            case 128: return launch_varlen_flags<128, true>(a, s);
            default: return hipErrorNotSupported;
        }
    }
    switch (a.DK) {
        case 32: return launch_varlen_flags<32, false>(a, s);
        case 64: return launch_varlen_flags<64, false>(a, s);
        case 128: return launch_varlen_flags<128, false>(a, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace gdn2
