// chunk_common.h -- device helpers shared by the chunkwise prefill kernels (gfx950).
#pragma once

#include "common.h"

namespace gdn2 {
namespace chunk {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length

// k-slot i of lane group g inside a 32-wide K-step, matching two stacked accumulator tiles:
// slots 0..3 are rows 4g..4g+3 of the first tile, slots 4..7 rows 4g..4g+3 of the second.
__device__ __forceinline__ int kap(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only. Waves exchange data through LDS alone, so global
// loads in flight (the next chunk's inputs) and global stores need not drain at a barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
// Logistic sigmoid, and log2 of it in a form that neither overflows nor cancels:
// log2 sigma(x) = min(x, 0) log2(e) - log2(1 + 2^(-|x| log2(e))). sigma(-inf) = 0, sigma(+inf) = 1.
// (the reciprocal is the hardware one, within 1 ulp: a gate needs no correctly rounded division)
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.f + ex2(-1.4426950408889634f * x)); }
__device__ __forceinline__ float lg2_sigmoid(float x) {
    return fminf(x, 0.f) * 1.4426950408889634f - lg2(1.f + ex2(-1.4426950408889634f * fabsf(x)));
}

// Raw buffer over [base, base + bytes): loads at byte offsets past the end return zero and
// stores there are dropped, so a ragged last chunk needs no branch (and the compiler can count
// the memory operations in flight exactly).
// Every caller passes a base and size that are the same in all lanes of the wavefront; reading
// them from the first active lane says so to the compiler, which otherwise may keep a descriptor
// it cannot prove uniform in vector registers and issue each access in a loop over its distinct
// values (one pass, but a loop that splits the code around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Raw buffer over token rows [r0, r0 + min(len - r0, maxrows)) of a sequence whose first token
// row is `first` in a tensor of row_bytes per token row. The base is advanced in 64-bit
// arithmetic, so a sequence may span more than 4 GiB; offsets inside stay below
// maxrows * row_bytes, and rows past the sequence end fall outside the buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, long first, long r0, long len,
                                                            unsigned row_bytes, int maxrows) {
    const long left = len - r0;
    const unsigned rows = left <= 0 ? 0u : (left < maxrows ? (unsigned)left : (unsigned)maxrows);
    return make_rsrc(static_cast<const char*>(base) + (first + r0) * (long)row_bytes, rows * row_bytes);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Cache policy of a buffer store (its aux operand): 0 is the default; kStreamStore sets sc1 and
// nt, the streaming policy, for outputs that no later kernel of the call reads back. Measured on
// the two-kernel prefill's o stores (B8 H16 T4096 d128): 0.4540 -> 0.4475 ms per call, outputs
// bit-equal; nt alone (0.4564) and sc1 alone (0.4576) were slower than the default.
constexpr int kStreamStore = 18;
template <int POL = 0>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, unsigned off, float a, float b, float c, float d) {
    const u32x4 x = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)off, 0, POL);
}

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

// ---- small helpers -------------------------------------------------------------------------

// Value of lane (l16 - N) within each row of 16 lanes, 0 for the first N lanes of the row.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xF, 0xF, true));
}

// Eight input elements of one row as loaded (packed bf16: one 16-byte vector; fp32: two).
template <bool BF16>
struct Raw8 {
    uint4 u[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> gload8(const void* base, long idx) {
    Raw8<BF16> r;
    if constexpr (BF16) {
        r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
        r.u[0] = p[0];
        r.u[1] = p[1];
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> fill8(float x) {
    Raw8<BF16> r;
    if constexpr (BF16) {
        const uint32_t h = __float_as_uint(x) >> 16;  // exact for 0, 1 and +-inf
        const uint32_t p = h | (h << 16);
        r.u[0] = make_uint4(p, p, p, p);
    } else {
        const uint32_t p = __float_as_uint(x);
        r.u[0] = r.u[1] = make_uint4(p, p, p, p);
    }
    return r;
}

// r where the row is valid, else eight copies of x. Loads are issued unconditionally (from a
// clamped, valid row) and replaced here at their first use: branch-free loads let the compiler
// count the loads in flight exactly and wait only for the ones a use needs.
template <bool BF16>
__device__ __forceinline__ Raw8<BF16> keep_or(const Raw8<BF16>& r, bool valid, float x) {
    const Raw8<BF16> f = fill8<BF16>(x);
    Raw8<BF16> o;
#pragma unroll
    for (int h = 0; h < (BF16 ? 1 : 2); ++h) {
        o.u[h].x = valid ? r.u[h].x : f.u[h].x;
        o.u[h].y = valid ? r.u[h].y : f.u[h].y;
        o.u[h].z = valid ? r.u[h].z : f.u[h].z;
        o.u[h].w = valid ? r.u[h].w : f.u[h].w;
    }
    return o;
}

template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float* x) {
    if constexpr (BF16) {
        const uint32_t w[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            x[4 * h + 0] = __uint_as_float(r.u[h].x);
            x[4 * h + 1] = __uint_as_float(r.u[h].y);
            x[4 * h + 2] = __uint_as_float(r.u[h].z);
            x[4 * h + 3] = __uint_as_float(r.u[h].w);
        }
    }
}

__device__ __forceinline__ void lds_read8f(const float* p, float* x) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Largest value over the wavefront: rotations within each row of 16 lanes (DPP row_ror), then the
// four row results read into scalars.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, row_ror<8>(x));
    x = fmaxf(x, row_ror<4>(x));
    x = fmaxf(x, row_ror<2>(x));
    x = fmaxf(x, row_ror<1>(x));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Range of the fp16 matrix-core operands. A chain wave holds its state columns times sc = 2^esc
// (the same for the wave) and multiplies this chunk's U = w v, the first operand it forms from
// them, by the same sc; D', Delta, O and the state update are then all times sc, and o and the
// final state are multiplied by isc = 2^-esc on the way out (exact: powers of two). Before the
// state and D' are rounded to fp16 for a chunk's products, esc is renewed when the wave's largest
// |S sc| or |U sc| leaves [2^-4, 2^8]: the new esc brings it to [2^3, 2^4). The upper end keeps
// E_hat S and the products after it far below fp16's largest finite value (65504) for gates in
// [0, 1] and keys of norm 1; the lower end keeps the state's leading digits out of fp16's
// subnormal range. esc stays within [-100, 100] (a state that has decayed below about 2^-96 along
// with its inputs is let go to fp16's subnormals and zero, where it no longer matters next to
// anything of normal size) and moves by at most 120 per chunk, so sc, isc and the step factor are
// finite normal floats. A non-finite maximum (a NaN in the inputs) leaves esc as it is.
// Sacc: the wave's state tiles (NMK 16-row tiles of its 16 columns); D: this chunk's U = w v rows
// in accumulator layout, multiplied by sc here.
template <int NMK>
__device__ __forceinline__ void rescale_state(f4 (&Sacc)[NMK], f4 (&D)[4], int& esc, float& sc, float& isc) {
    float ms = 0.f, mu = 0.f;
#pragma unroll
    for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
        for (int j = 0; j < 4; ++j) ms = fmaxf(ms, fabsf(Sacc[mk][j]));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mu = fmaxf(mu, fabsf(D[mt][j]));
    const float mm = wave_max(fmaxf(ms, mu * sc));
    if ((mm > 256.f && mm <= 3.0e38f) || (mm < 0.0625f && mm > 0.f)) {  // uniform over the wave
        const int e = __builtin_amdgcn_frexp_expf(mm);                  // mm in [2^(e-1), 2^e)
        const int step = min(max(4 - e, -120), 120);
        const int en = min(max(esc + step, -100), 100);
        if (en != esc) {
            const float r = __builtin_ldexpf(1.f, en - esc);
            esc = en;
            sc = __builtin_ldexpf(1.f, en);
            isc = __builtin_ldexpf(1.f, -en);
#pragma unroll
            for (int mk = 0; mk < NMK; ++mk)
#pragma unroll
                for (int j = 0; j < 4; ++j) Sacc[mk][j] *= r;
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) D[mt][j] *= sc;
}

// Per-(block, channel) decay tables, index t of tab[t][DK] (log2 domain, X = local value at a
// block's 8th row, G_I = sum of earlier block totals, gC = chunk total):
//   0..3 exp2(X_I)   4..7 exp2(G_I)   8..11 exp2(tot_I - X_I)   12..15 exp2(gC - G_{I+1})
//   16 exp2(gC)      17 exp2(tot_1)   18 exp2(tot_1 + tot_2)    19 exp2(tot_2)
constexpr int kTabs = 20;

}  // namespace chunk
}  // namespace gdn2
