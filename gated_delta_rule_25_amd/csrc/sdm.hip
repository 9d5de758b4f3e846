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
// Addressing (sdm_address_kernel): the two halves of each query are scored against their sub-key
// tables on the matrix cores (exact products, fp32 accumulation), 16 queries of a head at a time;
// then one wavefront per query selects: each half's best 64
// (score descending, equal scores: lower index first) come from bitonic sorts over the lanes of
// each 64-score column and merges of the sorted columns, all in registers. A pair of ranks (i, j)
// can be among the m best pair sums only if (i + 1)(j + 1) <= m (every pair of lower ranks in both
// halves precedes it), so only those pairs (280 for m = 64) are formed, reduced the same way
// (equal sums: lower slot first), and the first m are the slots i_sub * n + j_sub; their weights
// are the softmax of the sums.
//
// Update (sdm_fwd_kernel), one workgroup per (batch, head, 64 value columns), a lane per column:
// value columns do not interact, so each lane gathers its column of the W write slots and the R
// read slots in one round trip (the slots split over four wavefronts), forms e = a^T M, and
// writes the W updated entries back; a read slot that the token also writes takes the written
// value. The decay is a scalar
// on every slot, applied lazily: each slot carries the running sum of log alpha at its last
// write (fp64), and its value now is the stored one times exp(L - stamp). So a token reads and
// writes only its W + R slots and their stamps, never the whole memory.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

constexpr int kMaxSlots = 64;     // W, R and m at most one wavefront wide
constexpr float kFoldBelow = 0x1p-60f;

// Keys of the selection: (score, index) as one 64-bit integer whose ascending order is score
// descending, then index ascending (the total order of the oracle's selection): the score's bits
// mapped to an order-preserving unsigned integer and inverted, above the index.
__device__ __forceinline__ uint64_t sel_key(float s, int i) {
    const uint32_t u = __float_as_uint(s + 0.f);  // -0 counts as +0
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)(~asc) << 32) | (uint32_t)i;
}
__device__ __forceinline__ float key_score(uint64_t k) {
    const uint32_t asc = ~(uint32_t)(k >> 32);
    return __uint_as_float((asc & 0x80000000u) ? (asc & 0x7fffffffu) : ~asc);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)(uint32_t)k; }
constexpr uint64_t kNoKey = ~0ull;  // sorts after every real key

// x from lane (lane ^ j), j a power of two below 64 (a constant once the callers' loops unroll),
// without the LDS crossbar: DPP within rows of 16 lanes, the gfx950 permlane swaps across rows.
__device__ __forceinline__ uint32_t xor_lanes(uint32_t x, int j, int lane) {
    switch (j) {
        case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
        case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
        case 4: {
            const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x104, 0xF, 0xF, true);  // row_shl:4
            const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
            return (lane & 4) ? dn : up;
        }
        case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, true);   // row_ror:8
        case 15: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, true);  // row_mirror
        case 16: {  // odd rows of the first copy trade places with even rows of the second
            const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
            return (lane & 16) ? r[0] : r[1];
        }
        case 32: {  // upper half of the first copy trades places with lower half of the second
            const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
            return (lane & 32) ? r[0] : r[1];
        }
        default: return (uint32_t)__shfl_xor((int)x, j);
    }
}
__device__ __forceinline__ uint64_t xor_lanes64(uint64_t x, int j, int lane) {
    const uint32_t lo = xor_lanes((uint32_t)x, j, lane), hi = xor_lanes((uint32_t)(x >> 32), j, lane);
    return ((uint64_t)hi << 32) | lo;
}
// Ascending sort of NC columns of 64 keys (one key per lane and column) by a bitonic network over
// the lanes, the columns in lockstep so that their exchanges overlap. At each stage a lane keeps
// the smaller of its key and its partner's where `keep_min`, else the larger.
template <int NC>
__device__ __forceinline__ void sort64(uint64_t (&c)[NC], int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const bool keep_min = ((lane & j) == 0) == ((lane & k) == 0);
            uint64_t p[NC];
#pragma unroll
            for (int i = 0; i < NC; ++i) p[i] = xor_lanes64(c[i], j, lane);
#pragma unroll
            for (int i = 0; i < NC; ++i) c[i] = ((p[i] < c[i]) == keep_min) ? p[i] : c[i];
        }
}

// a[i] := the 64 smallest keys of the ascending 64-key lists a[i] and b[i], ascending: the lanewise
// minimum of a list and the other reversed is a bitonic sequence holding them, which one
// half-cleaner cascade sorts.
template <int NP>
__device__ __forceinline__ void merge64(uint64_t (&a)[NP], const uint64_t (&b)[NP], int lane) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const uint64_t rev = xor_lanes64(xor_lanes64(xor_lanes64(b[i], 15, lane), 16, lane), 32, lane);  // lane 63 - l
        a[i] = rev < a[i] ? rev : a[i];
    }
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
        const bool keep_min = (lane & j) == 0;
        uint64_t p[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) p[i] = xor_lanes64(a[i], j, lane);
#pragma unroll
        for (int i = 0; i < NP; ++i) a[i] = ((p[i] < a[i]) == keep_min) ? p[i] : a[i];
    }
}

// out[g] := the 64 smallest keys of the E sorted columns c[g][.], ascending (lane l holds rank l),
// by a tree of pairwise merges, the G groups in lockstep.
template <int G, int E>
__device__ __forceinline__ void best64(const uint64_t (&c)[G][E], uint64_t (&out)[G], int lane) {
    if constexpr (E == 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) out[g] = c[g][0];
    } else {
        constexpr int P = E / 2;
        uint64_t a[G * P], b[G * P];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < P; ++i) a[g * P + i] = c[g][2 * i], b[g * P + i] = c[g][2 * i + 1];
        merge64<G * P>(a, b, lane);
        uint64_t n[G][E - P];
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int i = 0; i < P; ++i) n[g][i] = a[g * P + i];
            if constexpr (E % 2 == 1) n[g][P] = c[g][E - 1];
        }
        best64<G, E - P>(n, out, lane);
    }
}

// Operand fragments of the score products on the matrix cores: lane (r, g) of a fragment holds
// the 8 consecutive channels 32 ks + 8 g .. + 7 of row r (a sub-key, or a query). bf16 runs as one
// 16x16x32 product; fp32 as eight 16x16x4 fp32 passes, pass i contracting slot i of every lane
// group. Both multiply exactly and accumulate in fp32.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <bool BF16>
struct ScoreFrag;
template <>
struct ScoreFrag<true> {
    bf16x8 v;
    __device__ void load(const void* base, long i) {
        v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i));
    }
    __device__ void zero() { v = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u)); }
    __device__ static void mma(f32x4& c, const ScoreFrag& a, const ScoreFrag& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
    }
};
template <>
struct ScoreFrag<false> {
    float v[8];
    __device__ void load(const void* base, long i) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
        const float4 lo = p[0], hi = p[1];
        v[0] = lo.x, v[1] = lo.y, v[2] = lo.z, v[3] = lo.w, v[4] = hi.x, v[5] = hi.y, v[6] = hi.z, v[7] = hi.w;
    }
    __device__ void zero() {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    __device__ static void mma(f32x4& c, const ScoreFrag& a, const ScoreFrag& b) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
    }
};

// A workgroup of four wavefronts takes 16 queries of one head at a time (grid-stride over
// (16-query tile, head)). The sub-key scores of both halves are 16 x 16 (sub-keys x queries) matrix
// core products into LDS, so each sub-key table is read once per tile, not once per query. Then
// each wavefront selects for 4 of the queries: lane l takes sub-keys l, l + 64, ... of each half;
// the best m of each half (ranks in lanes 0 .. m-1) come from the sorted columns and their merges;
// the candidate pairs, listed once per workgroup in LDS (slot c holds ranks (i, j)), are scored
// from the two rank lists by lane shuffles and reduced the same way.
constexpr int kCandCols = 5;  // 320 candidate slots: at most 280 pairs for m = 64
constexpr int kAddrQ = 16;    // queries per tile

template <int HALF, int NSUB, bool BF16>
__global__ void __launch_bounds__(256) sdm_address_kernel(const void* __restrict__ x, const void* __restrict__ C1,
                                                          const void* __restrict__ C2, long rows, int H, int m,
                                                          int* __restrict__ idx, float* __restrict__ wt) {
    constexpr int DK = 2 * HALF;
    constexpr int E = NSUB / 64;   // score columns per lane
    constexpr int KS = HALF / 32;  // 32-channel steps per half
    constexpr int LD = NSUB + 4;   // score row stride: rows start 4 banks apart
    static_assert(HALF % 32 == 0 && NSUB % 64 == 0, "tile shape");
    __shared__ float sc[2][kAddrQ][LD];
    __shared__ uint16_t cand[kCandCols * 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    // candidate pairs (i, j) with (i + 1)(j + 1) <= m: rank i contributes m / (i + 1) of them
    for (int c = tid; c < kCandCols * 64; c += 256) cand[c] = 0xffffu;
    __syncthreads();
    if (tid < m) {
        int c0 = 0;
        for (int i = 0; i < tid; ++i) c0 += m / (i + 1);
        const int cnt = m / (tid + 1);
        for (int j = 0; j < cnt; ++j) cand[c0 + j] = (uint16_t)((tid << 8) | j);
    }
    const long work = (rows + kAddrQ - 1) / kAddrQ * H;
#pragma unroll 1
    for (long wi = blockIdx.x; wi < work; wi += gridDim.x) {
        const int h = (int)(wi % H);
        const long r0 = wi / H * kAddrQ;
        // scores: sc[half][q][p] = <x_q half, C_half[h][p]>, fp32 accumulation
        const long rq = r0 + r16;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const void* C = half ? C2 : C1;
            ScoreFrag<BF16> xf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (rq < rows)
                    xf[ks].load(x, (rq * H + h) * DK + half * HALF + 32 * ks + 8 * g);
                else
                    xf[ks].zero();
            }
#pragma unroll 2
            for (int pb = wv; pb < NSUB / 16; pb += 4) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    ScoreFrag<BF16> cf;
                    cf.load(C, ((long)h * NSUB + pb * 16 + r16) * HALF + 32 * ks + 8 * g);
                    ScoreFrag<BF16>::mma(acc, cf, xf[ks]);
                }
                // acc[i]: sub-key pb * 16 + 4 g + i against query r16
                *reinterpret_cast<float4*>(&sc[half][r16][pb * 16 + 4 * g]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
        __syncthreads();
#pragma unroll 1
        for (int q = wv; q < kAddrQ && r0 + q < rows; q += 4) {
            const long qy = (r0 + q) * H + h;
            uint64_t col[2][E], top[2];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int e = 0; e < E; ++e) col[half][e] = sel_key(sc[half][q][64 * e + lane], 64 * e + lane);
            sort64<2 * E>(reinterpret_cast<uint64_t(&)[2 * E]>(col), lane);
            best64<2, E>(col, top, lane);
            // the candidate pairs' sums and slots, then the best m of them
            const float s1 = key_score(top[0]), s2 = key_score(top[1]);
            const int i1 = key_index(top[0]), i2 = key_index(top[1]);
            uint64_t cc[1][kCandCols], best[1];
#pragma unroll
            for (int u = 0; u < kCandCols; ++u) {
                const uint32_t ent = cand[64 * u + lane];
                const int ri = ent == 0xffffu ? 0 : (int)(ent >> 8), rj = ent == 0xffffu ? 0 : (int)(ent & 255u);
                const float a = __shfl(s1, ri), bsc = __shfl(s2, rj);
                const int slot = __shfl(i1, ri) * NSUB + __shfl(i2, rj);
                cc[0][u] = ent == 0xffffu ? kNoKey : sel_key(a + bsc, slot);
            }
            sort64<kCandCols>(cc[0], lane);
            best64<1, kCandCols>(cc, best, lane);
            // softmax of the m best sums (rank 0 is the largest)
            const float sb = key_score(best[0]);
            const float top0 = __shfl(sb, 0);
            const float ex = lane < m ? expf(sb - top0) : 0.f;
            float sum = ex;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
            if (lane < m) {
                idx[qy * m + lane] = key_index(best[0]);
                wt[qy * m + lane] = ex / sum;
            }
        }
        __syncthreads();  // sc is rewritten by the next tile
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

// One workgroup per (batch, head, 64 value columns), a lane per column; its four wavefronts each
// own 16 positions of the token's write list and 16 of its read list. The memory is kept in plain
// units per slot as of that slot's last write; stamp[s] holds the running sum of log alpha (fp64)
// at that write, and the slot's value now is M[s] * exp(L - stamp[s]). A token therefore touches
// only its W + R slots. Per token: each wavefront gathers its rows and stamps and forms its part
// of e = a^T M; the parts meet in LDS (summed in wavefront order); each wavefront writes its
// updated rows and forms its part of the read; a read slot that the token also writes is read
// from the writer's new value (its own gathered copy is weighted 0). The barrier that closes a
// token orders its row and stamp stores before every wavefront's next gathers. Each workgroup
// keeps its own stamps and L (the column tiles of a head run independently).
constexpr int kFwdWaves = 4;
constexpr int kPart = kMaxSlots / kFwdWaves;  // list positions per wavefront

template <bool BF16>
__global__ void __launch_bounds__(kFwdWaves * 64) sdm_fwd_kernel(
    const void* __restrict__ v, const void* __restrict__ alpha, const void* __restrict__ b, const void* __restrict__ w,
    const int* __restrict__ widx, const float* __restrict__ wwt, const int* __restrict__ ridx,
    const float* __restrict__ rwt, float* M, double* stamp, double* Lbuf, float* __restrict__ o, int T, int H, long N,
    int dv, int W, int R) {
    __shared__ float ep[kFwdWaves][kWave], op[kFwdWaves][kWave], rmp[kFwdWaves][kWave];
    __shared__ int ovp[kFwdWaves][kWave];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int tiles = dv / kWave;
    const long bh = blockIdx.x / tiles;
    const int tile = (int)(blockIdx.x % tiles);
    const int c = tile * kWave + lane;
    const long bb = bh / H;
    const int h = (int)(bh % H);
    float* Mb = M + bh * N * dv + c;
    double* Sb = stamp + (bh * tiles + tile) * N;
    double L = Lbuf[bh * tiles + tile];
    const int j0 = wv * kPart;  // this wavefront's list positions j0 .. j0 + kPart - 1
    const bool mine = lane >= j0 && lane < j0 + kPart;
    TokIn x = load_tok<BF16>(v, alpha, b, w, widx, wwt, ridx, rwt, (bb * T) * H + h, dv, c, W, R, lane);
#pragma unroll 1
    for (int t = 0; t < T; ++t) {
        const long tok = (bb * T + t) * H + h;
        // alpha = 0 wipes the memory: a decay of e^-1e6, zero in any float, keeps L finite
        L += x.al > 0.f ? log((double)x.al) : -1e6;
        const bool wok = (unsigned)x.wi < (unsigned long)N, rok = (unsigned)x.ri < (unsigned long)N;
        const double sw = (mine && wok) ? Sb[x.wi] : L, sr = (mine && rok) ? Sb[x.ri] : L;
        float mw[kPart], mr[kPart];
#pragma unroll
        for (int k = 0; k < kPart; ++k) {
            const int s = __builtin_amdgcn_readlane(x.wi, j0 + k);
            mw[k] = (j0 + k < W && (unsigned)s < (unsigned long)N) ? Mb[(long)s * dv] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kPart; ++k) {
            const int s = __builtin_amdgcn_readlane(x.ri, j0 + k);
            mr[k] = (j0 + k < R && (unsigned)s < (unsigned long)N) ? Mb[(long)s * dv] : 0.f;
        }
        TokIn nx = x;  // the next token's inputs, in flight meanwhile
        if (t + 1 < T) nx = load_tok<BF16>(v, alpha, b, w, widx, wwt, ridx, rwt, tok + H, dv, c, W, R, lane);
        // overlaps against this wavefront's positions of the other list: in lane r, whether read
        // slot r is written; in lane j, the read weight falling on write slot j
        int ovw = 0;
        float rmw = 0.f;
#pragma unroll
        for (int k = 0; k < kPart; ++k) {
            const int p = j0 + k;
            const int wp = __builtin_amdgcn_readlane(x.wi, p), rp = __builtin_amdgcn_readlane(x.ri, p);
            ovw |= (p < W) && rok && wp == x.ri;
            rmw += ((p < R) && wok && rp == x.wi) ? lane_f(x.ra, p) : 0.f;
        }
        ovp[wv][lane] = ovw;
        rmp[wv][lane] = rmw;
        // decay since each own slot's last write (slot j's factor in lane j)
        const float dw = (mine && wok) ? (float)exp(L - sw) : 0.f;
        const float dr = (mine && rok) ? (float)exp(L - sr) : 0.f;
        float e = 0.f;  // this wavefront's part of a^T (decayed M), in list order
#pragma unroll
        for (int k = 0; k < kPart; ++k) {
            mw[k] *= lane_f(dw, j0 + k);
            e = fmaf(lane_f(x.wa, j0 + k), mw[k], e);
        }
        ep[wv][lane] = e;
        __syncthreads();
        e = ep[0][lane];
        int ov = ovp[0][lane];
        float rmatch = rmp[0][lane];
#pragma unroll
        for (int q = 1; q < kFwdWaves; ++q) {
            e += ep[q][lane];
            ov |= ovp[q][lane];
            rmatch += rmp[q][lane];
        }
        const float u = x.ww * x.vv - x.be * e;
        const float rw = (rok && !ov) ? x.ra * dr : 0.f;  // read weight times decay; 0 where written
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < kPart; ++k) {
            const int s = __builtin_amdgcn_readlane(x.wi, j0 + k);
            const float nv = fmaf(lane_f(x.wa, j0 + k), u, mw[k]);
            if (j0 + k < W && (unsigned)s < (unsigned long)N) Mb[(long)s * dv] = nv;
            acc = fmaf(lane_f(rmatch, j0 + k), nv, acc);
        }
#pragma unroll
        for (int k = 0; k < kPart; ++k) acc = fmaf(lane_f(rw, j0 + k), mr[k], acc);
        if (mine && wok) Sb[x.wi] = L;
        op[wv][lane] = acc;
        __syncthreads();  // also orders this token's row and stamp stores before the next gathers
        if (wv == 0) {
            float oc = op[0][lane];
#pragma unroll
            for (int q = 1; q < kFwdWaves; ++q) oc += op[q][lane];
            o[tok * dv + c] = oc;
        }
        x = nx;
    }
    if (threadIdx.x == 0) Lbuf[bh * tiles + tile] = L;
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
hipError_t launch_address_n(const SdmAddressArgs& a, hipStream_t st, int grid, long rows) {
    switch (a.n) {
        case 64: hipLaunchKernelGGL((sdm_address_kernel<HALF, 64, BF16>), dim3(grid), dim3(256), 0, st, a.x, a.C1, a.C2, rows, a.H, a.m, a.idx, a.wt); break;
        case 128: hipLaunchKernelGGL((sdm_address_kernel<HALF, 128, BF16>), dim3(grid), dim3(256), 0, st, a.x, a.C1, a.C2, rows, a.H, a.m, a.idx, a.wt); break;
        case 256: hipLaunchKernelGGL((sdm_address_kernel<HALF, 256, BF16>), dim3(grid), dim3(256), 0, st, a.x, a.C1, a.C2, rows, a.H, a.m, a.idx, a.wt); break;
        case 512: hipLaunchKernelGGL((sdm_address_kernel<HALF, 512, BF16>), dim3(grid), dim3(256), 0, st, a.x, a.C1, a.C2, rows, a.H, a.m, a.idx, a.wt); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_address_t(const SdmAddressArgs& a, hipStream_t st) {
    const long rows = a.queries / a.H;
    const long work = (rows + kAddrQ - 1) / kAddrQ * a.H;       // (16-query tile, head) pairs
    const int grid = (int)(work < 256L * 32 ? work : 256L * 32);  // grid-stride beyond 32 per CU
    switch (a.dk) {
        case 64: return launch_address_n<32, BF16>(a, st, grid, rows);
        case 128: return launch_address_n<64, BF16>(a, st, grid, rows);
        case 256: return launch_address_n<128, BF16>(a, st, grid, rows);
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
        hipLaunchKernelGGL((sdm_fwd_kernel<true>), dim3((unsigned)grid), dim3(kFwdWaves * 64), 0, st, a.v, a.alpha, a.b, a.w, a.widx,
                           a.wwt, a.ridx, a.rwt, a.M, a.stamp, a.L, a.o, a.T, a.H, a.N, a.dv, a.W, a.R);
    else
        hipLaunchKernelGGL((sdm_fwd_kernel<false>), dim3((unsigned)grid), dim3(kFwdWaves * 64), 0, st, a.v, a.alpha, a.b, a.w, a.widx,
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
