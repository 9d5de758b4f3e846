// common.h -- small device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

constexpr int kWave = 64;  // CDNA wavefront width

// bfloat16 bit pattern -> float (exact: bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) {
    return __uint_as_float(pair & 0xffff0000u);
}

// Load N contiguous input elements (bf16 or fp32) starting at element `idx` of `base` and
// widen them to fp32. The caller guarantees the address is aligned to the vector width used:
// 8*N bytes up to 16 for bf16 groups of 4/8, 16 bytes for fp32 groups of 4.
template <int N, bool BF16>
__device__ __forceinline__ void load_vec(const void* base, long idx, float* out) {
    static_assert(N % 4 == 0, "N must be a multiple of 4");
    if constexpr (BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + idx;
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N / 8; ++i) {
                const uint4 u = reinterpret_cast<const uint4*>(p)[i];
                out[8 * i + 0] = bf16_lo(u.x);
                out[8 * i + 1] = bf16_hi(u.x);
                out[8 * i + 2] = bf16_lo(u.y);
                out[8 * i + 3] = bf16_hi(u.y);
                out[8 * i + 4] = bf16_lo(u.z);
                out[8 * i + 5] = bf16_hi(u.z);
                out[8 * i + 6] = bf16_lo(u.w);
                out[8 * i + 7] = bf16_hi(u.w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < N / 4; ++i) {
                const uint2 u = reinterpret_cast<const uint2*>(p)[i];
                out[4 * i + 0] = bf16_lo(u.x);
                out[4 * i + 1] = bf16_hi(u.x);
                out[4 * i + 2] = bf16_lo(u.y);
                out[4 * i + 3] = bf16_hi(u.y);
            }
        }
    } else {
        const float* p = static_cast<const float*>(base) + idx;
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const float4 f = reinterpret_cast<const float4*>(p)[i];
            out[4 * i + 0] = f.x;
            out[4 * i + 1] = f.y;
            out[4 * i + 2] = f.z;
            out[4 * i + 3] = f.w;
        }
    }
}

// One input element widened to fp32.
template <bool BF16>
__device__ __forceinline__ float load_one(const void* base, long idx) {
    if constexpr (BF16) {
        return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    } else {
        return static_cast<const float*>(base)[idx];
    }
}

}  // namespace gdn2
