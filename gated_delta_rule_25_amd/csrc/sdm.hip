// sdm.hip -- sparse delta memory (SDM) kernels for gfx950: product-key slot addressing and the
// token-by-token sparse Gated DeltaNet-2 update of a large slot memory.
//
// Method: the aiweekly.co article "Meta FAIR dévoile SDM, un RNN linéaire à mémoire sparse
// massive" (second paragraph: Gated DeltaNet with the dense key-value outer product replaced by
// sparse reads and writes into a large memory; a product-key index picks W write and R read
// slots out of N per token, W = R = 64), applied to the update of the page "NVIDIA представила
// Gated DeltaNet-2 ...", paragraph "Техническая схема", with the key replaced by the sparse
// N-vector a of write weights:
//     M_t = (I - b_t a a^T) alpha_t M_{t-1} + a (w_t * v_t)^T,   o_t = M_t^T r,
// alpha_t and b_t per-token scalars (they act on the slot axis), w_t on the value axis, r the
// sparse read weights.
//
// Addressing (sdm_address_kernel), one wavefront per query: the two halves of the query are
// scored against their sub-key tables (fp32 dot products in channel order); each half's n scores
// are sorted by a bitonic network in LDS (score descending, equal scores: lower index first) and
// the first m kept. A pair of ranks (i, j) can be among the m best pair sums only if
// (i + 1)(j + 1) <= m (every pair of lower ranks in both halves precedes it), so only those pairs
// (280 for m = 64) are formed, sorted the same way (equal sums: lower slot first), and the first
// m are the slots i_sub * n + j_sub; their weights are the softmax of the sums.
//
// Update (sdm_fwd_kernel), one wavefront per (batch, head, 64 value columns), a lane per column:
// value columns do not interact, so each lane gathers its column of the W write slots and the R
// read slots in one round trip, forms e = a^T M, and writes the W updated entries back; a read
// slot that the token also writes takes the written value from registers. The decay is a scalar
// on every slot, applied lazily: each slot carries the running sum of log alpha at its last
// write (fp64), and its value now is the stored one times exp(L - stamp). So a token reads and
// writes only its W + R slots and their stamps, never the whole memory.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

constexpr int kMaxSlots = 64;     // W, R and m at most one wavefront wide
constexpr int kCand = 512;        // candidate pairs (at most 280 for m = 64), padded for the sort
constexpr float kFoldBelow = 0x1p-60f;

// Total order of (score, index) keys: higher score first, equal scores lower index first.
__device__ __forceinline__ bool before(float sa, int ia, float sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// Sorts P keys held in LDS (ks, ki) into the order `before` defines, with a bitonic network run
// by the workgroup's single wavefront. P is a power of two.
template <int P>
__device__ __forceinline__ void wave_sort(float* ks, int* ki, int lane) {
#pragma unroll 1
    for (int k = 2; k <= P; k <<= 1) {
#pragma unroll 1
        for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
            for (int t = lane; t < P / 2; t += kWave) {
                const int i = (t / j) * 2 * j + (t % j), l = i + j;
                const float si = ks[i], sl = ks[l];
                const int ii = ki[i], il = ki[l];
                // ascending runs (in `before` order) where bit k of i is clear
                const bool swap = ((i & k) == 0) ? before(sl, il, si, ii) : before(si, ii, sl, il);
                if (swap) {
                    ks[i] = sl;
                    ks[l] = si;
                    ki[i] = il;
                    ki[l] = ii;
                }
            }
            __syncthreads();
        }
    }
}

template <int HALF, int NSUB, bool BF16>
__global__ void __launch_bounds__(64) sdm_address_kernel(const void* __restrict__ x, const void* __restrict__ C1,
                                                         const void* __restrict__ C2, long queries, int H, int m,
                                                         int* __restrict__ idx, float* __restrict__ wt) {
    constexpr int DK = 2 * HALF;
    __shared__ float xs[DK];
    __shared__ float ks[NSUB > kCand ? NSUB : kCand];
    __shared__ int ki[NSUB > kCand ? NSUB : kCand];
    __shared__ float top_s[2][kMaxSlots];
    __shared__ int top_i[2][kMaxSlots];
    __shared__ int cstart[kMaxSlots + 1];
    const int lane = threadIdx.x;
#pragma unroll 1
    for (long qy = blockIdx.x; qy < queries; qy += gridDim.x) {
        const int h = (int)(qy % H);
        for (int d = lane; d < DK; d += kWave) xs[d] = load_one<BF16>(x, qy * DK + d);
        __syncthreads();
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
            const void* C = half ? C2 : C1;
            const long row0 = (long)h * NSUB;
            for (int p = lane; p < NSUB; p += kWave) {  // score of sub-key p: fp32, channel order
                float s = 0.f;
#pragma unroll
                for (int d0 = 0; d0 < HALF; d0 += 8) {
                    float c[8];
                    load_vec<8, BF16>(C, (row0 + p) * HALF + d0, c);
#pragma unroll
                    for (int u = 0; u < 8; ++u) s = fmaf(c[u], xs[half * HALF + d0 + u], s);
                }
                ks[p] = s;
                ki[p] = p;
            }
            __syncthreads();
            wave_sort<NSUB>(ks, ki, lane);
            if (lane < m) {
                top_s[half][lane] = ks[lane];
                top_i[half][lane] = ki[lane];
            }
            __syncthreads();
        }
        // candidate pairs (i, j) with (i + 1)(j + 1) <= m: row i holds m / (i + 1) of them
        if (lane == 0) {
            int acc = 0;
            for (int i = 0; i < m; ++i) {
                cstart[i] = acc;
                acc += m / (i + 1);
            }
            cstart[m] = acc;
        }
        for (int c = lane; c < kCand; c += kWave) {  // padding sorts last
            ks[c] = -__builtin_inff();
            ki[c] = 0x7fffffff;
        }
        __syncthreads();
        if (lane < m) {
            const int c0 = cstart[lane], cnt = m / (lane + 1);
            const float a = top_s[0][lane];
            const int ia = top_i[0][lane];
            for (int j = 0; j < cnt; ++j) {
                ks[c0 + j] = a + top_s[1][j];
                ki[c0 + j] = ia * NSUB + top_i[1][j];
            }
        }
        __syncthreads();
        wave_sort<kCand>(ks, ki, lane);
        // softmax of the m best sums (the first is the largest)
        const float best = ks[0];
        const float e = lane < m ? expf(ks[lane] - best) : 0.f;
        float sum = e;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane < m) {
            idx[qy * m + lane] = ki[lane];
            wt[qy * m + lane] = e / sum;
        }
        __syncthreads();  // LDS is reused by the next query
    }
}

// Inputs of one token for one lane: the token's scalars and value entries, and slot j of the
// write and read lists in lane j.
struct TokIn {
    float al, be, vv, ww;
    int wi, ri;
    float wa, ra;
};

template <bool BF16>
__device__ __forceinline__ TokIn load_tok(const void* v, const void* alpha, const void* b, const void* w,
                                          const int* widx, const float* wwt, const int* ridx, const float* rwt,
                                          long tok, int dv, int c, int W, int R, int lane) {
    TokIn x;
    x.al = load_one<BF16>(alpha, tok);
    x.be = load_one<BF16>(b, tok);
    x.vv = load_one<BF16>(v, tok * dv + c);
    x.ww = w ? load_one<BF16>(w, tok * dv + c) : 1.f;
    x.wi = lane < W ? widx[tok * W + lane] : -1;
    x.wa = lane < W ? wwt[tok * W + lane] : 0.f;
    x.ri = lane < R ? ridx[tok * R + lane] : -1;
    x.ra = lane < R ? rwt[tok * R + lane] : 0.f;
    return x;
}

__device__ __forceinline__ float lane_f(float x, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}

// One wavefront per (batch, head, 64 value columns), a lane per column. The memory is kept in
// plain units per slot as of that slot's last write; stamp[s] holds the running sum of log alpha
// (fp64) at that write, and the slot's value now is M[s] * exp(L - stamp[s]). A token therefore
// touches only its W + R slots. Each wavefront keeps its own stamps and L (the column tiles of a
// head run independently), so no wavefront reads another's bookkeeping.
template <bool BF16>
__global__ void __launch_bounds__(64) sdm_fwd_kernel(const void* __restrict__ v, const void* __restrict__ alpha,
                                                     const void* __restrict__ b, const void* __restrict__ w,
                                                     const int* __restrict__ widx, const float* __restrict__ wwt,
                                                     const int* __restrict__ ridx, const float* __restrict__ rwt,
                                                     float* M, double* stamp, double* Lbuf, float* __restrict__ o,
                                                     int T, int H, long N, int dv, int W, int R) {
    const int lane = threadIdx.x;
    const int tiles = dv / kWave;
    const long bh = blockIdx.x / tiles;
    const int tile = (int)(blockIdx.x % tiles);
    const int c = tile * kWave + lane;
    const long bb = bh / H;
    const int h = (int)(bh % H);
    float* Mb = M + bh * N * dv + c;
    double* Sb = stamp + (bh * tiles + tile) * N;
    double L = Lbuf[bh * tiles + tile];
    TokIn x = load_tok<BF16>(v, alpha, b, w, widx, wwt, ridx, rwt, (bb * T) * H + h, dv, c, W, R, lane);
#pragma unroll 1
    for (int t = 0; t < T; ++t) {
        const long tok = (bb * T + t) * H + h;
        // alpha = 0 wipes the memory: a decay of e^-1e6, zero in any float, keeps L finite
        L += x.al > 0.f ? log((double)x.al) : -1e6;
        const bool wok = (unsigned)x.wi < (unsigned long)N, rok = (unsigned)x.ri < (unsigned long)N;
        // read slots this token also writes take the written value (held in registers below);
        // rmatch: the read weight that falls on this lane's write slot
        bool ov = false;
        float rmatch = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) {
            const int wj = __builtin_amdgcn_readlane(x.wi, j), rj = __builtin_amdgcn_readlane(x.ri, j);
            ov |= (j < W) && rok && wj == x.ri;
            rmatch += ((j < R) && wok && rj == x.wi) ? lane_f(x.ra, j) : 0.f;
        }
        const bool rload = rok && !ov;
        const double sw = wok ? Sb[x.wi] : L, sr = rload ? Sb[x.ri] : L;
        float mw[kMaxSlots], mr[kMaxSlots];
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) {
            const int s = __builtin_amdgcn_readlane(x.wi, j);
            mw[j] = (j < W && (unsigned)s < (unsigned long)N) ? Mb[(long)s * dv] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) {
            const int s = __builtin_amdgcn_readlane(x.ri, j);
            const bool ld = __builtin_amdgcn_readlane((int)rload, j) != 0;
            mr[j] = (j < R && ld) ? Mb[(long)s * dv] : 0.f;
        }
        TokIn nx = x;  // the next token's inputs, in flight meanwhile
        if (t + 1 < T) nx = load_tok<BF16>(v, alpha, b, w, widx, wwt, ridx, rwt, tok + H, dv, c, W, R, lane);
        // decay since each slot's last write (slot j's factor in lane j)
        const float dw = wok ? (float)exp(L - sw) : 0.f;
        const float dr = rload ? (float)exp(L - sr) : 0.f;
        float e = 0.f;  // a^T (decayed M) over the write slots, in slot order
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) {
            mw[j] *= lane_f(dw, j);
            e = fmaf(lane_f(x.wa, j), mw[j], e);
        }
        const float u = x.ww * x.vv - x.be * e;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) {
            const int s = __builtin_amdgcn_readlane(x.wi, j);
            const float nv = fmaf(lane_f(x.wa, j), u, mw[j]);
            if (j < W && (unsigned)s < (unsigned long)N) Mb[(long)s * dv] = nv;
            acc = fmaf(lane_f(rmatch, j), nv, acc);
        }
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) acc = fmaf(lane_f(x.ra, j) * lane_f(dr, j), mr[j], acc);
        o[tok * dv + c] = acc;
        if (wok) Sb[x.wi] = L;
        x = nx;
    }
    if (lane == 0) Lbuf[bh * tiles + tile] = L;
}

// M[s] *= exp(L - stamp[s]) for every slot, then stamp = L: the memory in plain units as of the
// last token. One workgroup per (batch, head, column tile, block of slots); each wavefront takes
// whole rows (its 64 lanes the row's 64 columns of the tile), so every lane has read a row's
// stamp before lane 0 rewrites it.
__global__ void __launch_bounds__(256) sdm_fold_kernel(float* M, double* stamp, const double* __restrict__ Lbuf,
                                                       long N, int dv, long blocks_per_tile) {
    const int tiles = dv / kWave;
    const long bt = blockIdx.x / blocks_per_tile;  // (batch * head) * tiles + tile
    const long blk = blockIdx.x % blocks_per_tile;
    const long bh = bt / tiles;
    const int tile = (int)(bt % tiles);
    const double L = Lbuf[bt];
    double* Sb = stamp + bt * N;
    float* Mb = M + bh * N * dv + tile * kWave;
    const int col = threadIdx.x % kWave;
    for (long s = blk * 4 + threadIdx.x / kWave; s < N; s += blocks_per_tile * 4) {
        const double st = Sb[s];
        Mb[s * dv + col] *= (float)exp(L - st);
        if (col == 0) Sb[s] = L;
    }
}

template <int HALF, bool BF16>
hipError_t launch_address_n(const SdmAddressArgs& a, hipStream_t st, int grid) {
    switch (a.n) {
        case 64: hipLaunchKernelGGL((sdm_address_kernel<HALF, 64, BF16>), dim3(grid), dim3(64), 0, st, a.x, a.C1, a.C2, a.queries, a.H, a.m, a.idx, a.wt); break;
        case 128: hipLaunchKernelGGL((sdm_address_kernel<HALF, 128, BF16>), dim3(grid), dim3(64), 0, st, a.x, a.C1, a.C2, a.queries, a.H, a.m, a.idx, a.wt); break;
        case 256: hipLaunchKernelGGL((sdm_address_kernel<HALF, 256, BF16>), dim3(grid), dim3(64), 0, st, a.x, a.C1, a.C2, a.queries, a.H, a.m, a.idx, a.wt); break;
        case 512: hipLaunchKernelGGL((sdm_address_kernel<HALF, 512, BF16>), dim3(grid), dim3(64), 0, st, a.x, a.C1, a.C2, a.queries, a.H, a.m, a.idx, a.wt); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_address_t(const SdmAddressArgs& a, hipStream_t st) {
    const long want = a.queries;
    const int grid = (int)(want < 256L * 64 ? want : 256L * 64);  // grid-stride beyond 64 waves per CU
    switch (a.dk) {
        case 64: return launch_address_n<32, BF16>(a, st, grid);
        case 128: return launch_address_n<64, BF16>(a, st, grid);
        case 256: return launch_address_n<128, BF16>(a, st, grid);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

bool sdm_address_supported(int dk, int n, int m) {
    return (dk == 64 || dk == 128 || dk == 256) && (n == 64 || n == 128 || n == 256 || n == 512) && m >= 1 &&
           m <= kMaxSlots && m <= n;
}

bool sdm_fwd_supported(int dv, int W, int R) {
    return (dv == 64 || dv == 128 || dv == 256) && W >= 1 && W <= kMaxSlots && R >= 1 && R <= kMaxSlots;
}

hipError_t launch_sdm_address(const SdmAddressArgs& a, hipStream_t st) {
    if (a.queries == 0) return hipSuccess;
    return a.bf16 ? launch_address_t<true>(a, st) : launch_address_t<false>(a, st);
}

hipError_t launch_sdm_fwd(const SdmFwdArgs& a, hipStream_t st) {
    if (a.T == 0 || a.B == 0) return hipSuccess;
    const long grid = (long)a.B * a.H * (a.dv / kWave);
    if (a.bf16)
        hipLaunchKernelGGL((sdm_fwd_kernel<true>), dim3((unsigned)grid), dim3(64), 0, st, a.v, a.alpha, a.b, a.w, a.widx,
                           a.wwt, a.ridx, a.rwt, a.M, a.stamp, a.L, a.o, a.T, a.H, a.N, a.dv, a.W, a.R);
    else
        hipLaunchKernelGGL((sdm_fwd_kernel<false>), dim3((unsigned)grid), dim3(64), 0, st, a.v, a.alpha, a.b, a.w, a.widx,
                           a.wwt, a.ridx, a.rwt, a.M, a.stamp, a.L, a.o, a.T, a.H, a.N, a.dv, a.W, a.R);
    return hipGetLastError();
}

hipError_t launch_sdm_fold(float* M, double* stamp, double* L, long heads, long N, int dv, hipStream_t st) {
    if (heads == 0) return hipSuccess;
    long bpt = (N + 3) / 4;  // blocks per (head, tile): 4 rows per block and step
    if (bpt > 64) bpt = 64;
    const long grid = heads * (dv / kWave) * bpt;
    hipLaunchKernelGGL(sdm_fold_kernel, dim3((unsigned)grid), dim3(256), 0, st, M, stamp, L, N, dv, bpt);
    return hipGetLastError();
}

}  // namespace gdn2
