// rmsnorm.hip -- the RMS normalisation the recurrent layer's output passes through [page "NVIDIA
// представила Gated DeltaNet-2 с канал-wise гейтами …", paragraph "Архитектурно"]: per row of D
// values (one head's d_v outputs of one token), y = x / sqrt(mean(x^2) + eps) * weight, and its
// backward.
//
// Both directions are one pass over HBM. A group of D/4 lanes owns a row, one 16-byte load per
// lane (a wavefront covers 64/(D/4) rows per load), and the row's sum is a butterfly inside the
// group. The backward's weight gradient, a sum over every row, is reduced deterministically:
// each workgroup sums its rows into a [D] partial in the workspace, then one pass adds the
// partials in workgroup order.
#include <mutex>

#include "kernels.h"

namespace gdn2 {

namespace {

constexpr int kNormBlocks = 1024;  // workgroups of the backward (and partials of dweight)

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ uint32_t bf16_rne(float f) {  // round to nearest even (finite inputs)
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {  // over the LPR lanes of a row group
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// x and y are not __restrict__: y may be x (in place, fp32); each lane loads its four elements
// before it stores the same four.
template <int D, bool BF16OUT>
__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(const float* x, const float* __restrict__ wt, void* y,
                                                          long rows, float eps) {
    constexpr int LPR = D / 4, RPB = 256 / LPR;  // lanes per row, rows per workgroup
    const int c = (threadIdx.x % LPR) * 4;
    const long r = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const bool live = r < rows;  // groups are row-aligned: a group is all live or all not
    const float4 v = live ? ld4(x + r * D + c) : float4{0.f, 0.f, 0.f, 0.f};
    const float ss = group_sum<LPR>(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
    const float s = 1.f / sqrtf(ss * (1.f / D) + eps);
    const float4 g = wt ? ld4(wt + c) : float4{1.f, 1.f, 1.f, 1.f};
    const float4 o{v.x * s * g.x, v.y * s * g.y, v.z * s * g.z, v.w * s * g.w};
    if (!live) return;
    if constexpr (BF16OUT) {
        uint2 p;
        p.x = bf16_rne(o.x) | (bf16_rne(o.y) << 16);
        p.y = bf16_rne(o.z) | (bf16_rne(o.w) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + r * D + c) = p;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + r * D + c) = o;
    }
}

// dx = s (u - xh mean(xh u)) with s = (mean(x^2) + eps)^(-1/2), xh = x s, u = dy * weight; the
// workgroup's sum of dy * xh over its rows goes to part[blockIdx][D] (when part is given). Each
// step of the grid-stride loop takes kUnroll row groups, all loaded before the first sum.
constexpr int kUnroll = 4;

template <int D>
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const float* __restrict__ x, const float* __restrict__ wt,
                                                          const float* dy, float* dx, float* __restrict__ part,
                                                          long rows, float eps) {
    constexpr int LPR = D / 4, RPB = 256 / LPR;
    __shared__ float4 red[256];
    const int c = (threadIdx.x % LPR) * 4;
    const float4 g = wt ? ld4(wt + c) : float4{1.f, 1.f, 1.f, 1.f};
    const float4 z{0.f, 0.f, 0.f, 0.f};
    float4 acc = z;
    for (long r0 = (long)blockIdx.x * RPB * kUnroll; r0 < rows; r0 += (long)gridDim.x * RPB * kUnroll) {
        float4 v[kUnroll], d[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const long r = r0 + j * RPB + threadIdx.x / LPR;
            v[j] = r < rows ? ld4(x + r * D + c) : z;
            d[j] = r < rows ? ld4(dy + r * D + c) : z;
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const long r = r0 + j * RPB + threadIdx.x / LPR;
            const float4 a = v[j], e = d[j];
            const float ss = group_sum<LPR>(a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w);
            // rows past the end (x = dy = 0) take s = 0, so that they add nothing to the weight
            // gradient even when eps = 0 (where 1 / sqrt(0) would make 0 * inf = NaN)
            const float s = r < rows ? 1.f / sqrtf(ss * (1.f / D) + eps) : 0.f;
            const float4 xh{a.x * s, a.y * s, a.z * s, a.w * s};
            const float4 u{e.x * g.x, e.y * g.y, e.z * g.z, e.w * g.w};
            const float m = group_sum<LPR>(xh.x * u.x + xh.y * u.y + xh.z * u.z + xh.w * u.w) * (1.f / D);
            acc.x = fmaf(e.x, xh.x, acc.x);
            acc.y = fmaf(e.y, xh.y, acc.y);
            acc.z = fmaf(e.z, xh.z, acc.z);
            acc.w = fmaf(e.w, xh.w, acc.w);
            if (r < rows)
                *reinterpret_cast<float4*>(dx + r * D + c) = float4{s * fmaf(-xh.x, m, u.x), s * fmaf(-xh.y, m, u.y),
                                                                    s * fmaf(-xh.z, m, u.z), s * fmaf(-xh.w, m, u.w)};
        }
    }
    if (!part) return;  // uniform over the workgroup
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < LPR) {  // column group c: the sum over the workgroup's RPB row groups
        float4 t = z;
        for (int j = 0; j < RPB; ++j) {
            const float4 a = red[j * LPR + threadIdx.x];
            t.x += a.x;
            t.y += a.y;
            t.z += a.z;
            t.w += a.w;
        }
        *reinterpret_cast<float4*>(part + (size_t)blockIdx.x * D + c) = t;
    }
}

// dweight[c] = the sum of the nblk partials, in a fixed order: a workgroup per 4 columns; thread
// (i, q) sums the partials j = i, i + 64, ... of column 4 blockIdx + q, then the 64 sums of a
// column are added in LDS as a fixed tree.
__global__ void __launch_bounds__(256) rmsnorm_wsum_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                           int nblk, int D) {
    __shared__ float red[256];
    const int q = threadIdx.x & 3, i = threadIdx.x >> 2, col = blockIdx.x * 4 + q;
    float t = 0.f;
    if (col < D)
        for (int j = i; j < nblk; j += 64) t += part[(size_t)j * D + col];
    red[threadIdx.x] = t;
    __syncthreads();
    for (int h = 32; h >= 1; h >>= 1) {  // red[4 i + q] += red[4 (i + h) + q] for i < h
        if (i < h) red[threadIdx.x] += red[threadIdx.x + 4 * h];
        __syncthreads();
    }
    if (i == 0 && col < D) dw[col] = red[q];
}

int bwd_blocks(long rows, int D) {
    const long rpb = 256 / (D / 4) * kUnroll;  // rows per step of a workgroup
    const long need = (rows + rpb - 1) / rpb;
    return (int)(need < kNormBlocks ? need : kNormBlocks);
}

template <int D>
hipError_t launch_fwd_t(const RmsNormArgs& a, hipStream_t st) {
    constexpr int RPB = 256 / (D / 4);
    if (a.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.rows + RPB - 1) / RPB));
    if (a.y_bf16)
        hipLaunchKernelGGL((rmsnorm_fwd_kernel<D, true>), grid, dim3(256), 0, st, a.x, a.weight, a.y, a.rows, a.eps);
    else
        hipLaunchKernelGGL((rmsnorm_fwd_kernel<D, false>), grid, dim3(256), 0, st, a.x, a.weight, a.y, a.rows, a.eps);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_t(const RmsNormArgs& a, hipStream_t st) {
    const int nblk = bwd_blocks(a.rows, D);
    float* part = a.dweight ? static_cast<float*>(a.workspace) : nullptr;
    if (nblk > 0)
        hipLaunchKernelGGL((rmsnorm_bwd_kernel<D>), dim3(nblk), dim3(256), 0, st, a.x, a.weight, a.dy, a.dx, part,
                           a.rows, a.eps);
    if (a.dweight)  // no rows: nblk = 0 and dweight = 0
        hipLaunchKernelGGL(rmsnorm_wsum_kernel, dim3((D + 3) / 4), dim3(256), 0, st, part, a.dweight, nblk, D);
    return hipGetLastError();
}

template <bool BWD>
hipError_t dispatch(const RmsNormArgs& a, hipStream_t s) {
    switch (a.D) {
        case 32: return BWD ? launch_bwd_t<32>(a, s) : launch_fwd_t<32>(a, s);
        case 64: return BWD ? launch_bwd_t<64>(a, s) : launch_fwd_t<64>(a, s);
        case 128: return BWD ? launch_bwd_t<128>(a, s) : launch_fwd_t<128>(a, s);
        case 256: return BWD ? launch_bwd_t<256>(a, s) : launch_fwd_t<256>(a, s);
        default: return hipErrorNotSupported;
    }
}

// Fixed scratch for callers that cannot allocate: the dweight partials of one backward call,
// at most kNormBlocks rows of D <= 256 floats (1 MiB). Each GPU holds its own copy of the array
// for the life of the process. In host code its name is a host-side stand-in, so the device
// address is looked up once per device and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = (size_t)kNormBlocks * 256 * sizeof(float);
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

}  // namespace

size_t rmsnorm_bwd_workspace_bytes(long rows, int D) { return (size_t)bwd_blocks(rows, D) * D * 4; }

hipError_t rmsnorm_scratch(void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {  // first call on this device: it is the current one
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_addr[dev] = p;
    }
    *ptr = scratch_addr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

hipError_t launch_rmsnorm_fwd(const RmsNormArgs& a, hipStream_t s) { return dispatch<false>(a, s); }
hipError_t launch_rmsnorm_bwd(const RmsNormArgs& a, hipStream_t s) { return dispatch<true>(a, s); }

}  // namespace gdn2
