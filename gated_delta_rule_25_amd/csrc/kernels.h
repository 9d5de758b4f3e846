// kernels.h -- internal launch interfaces between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

// Arguments of the token-by-token kernel (also the decode step: T = 1, S0 == S_out).
struct RecurrentArgs {
    const void *q, *k, *v, *alpha, *b, *w;
    const float* S0;
    float* o;
    float* S_out;
    int B, T, H, DK, DV;
    bool bf16;
    uint32_t flags;
};
hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s);

// Arguments of the chunkwise (C = 64) prefill kernels.
struct ChunkArgs {
    const void *q, *k, *v, *alpha, *b, *w;
    const float* S0;
    float* o;
    float* S_out;
    int B, T, H, DK, DV;
    bool bf16;
    uint32_t flags;
    void* workspace;
    size_t workspace_bytes;
};
// Returns hipErrorNotSupported when no chunk kernel covers the arguments.
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t s);
size_t chunk_workspace_bytes(int B, int T, int H, int DK, int DV, bool bf16, uint32_t flags);
bool chunk_supported(int DK, int DV, bool bf16);

}  // namespace gdn2
