// chunk.hip -- chunkwise (C = 64) prefill kernels. (Kernels not written yet.)
#include "common.h"
#include "kernels.h"

namespace gdn2 {

bool chunk_supported(int DK, int DV, bool bf16) { return false; }

size_t chunk_workspace_bytes(int B, int T, int H, int DK, int DV, bool bf16, uint32_t flags) {
    return 0;
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t s) { return hipErrorNotSupported; }

}  // namespace gdn2
