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
    const int* slots = nullptr;  // decode over a state pool: batch row b uses state slots[b]
    int n_slots = 0;
};
hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s);

// Output RMS normalisation per row of D values (D in {32, 64, 128, 256}).
struct RmsNormArgs {
    const float* x;
    const float* weight;  // [D] or null (ones)
    void* y;              // forward: [rows, D], fp32 or bf16
    bool y_bf16;
    const float* dy;  // backward: [rows, D] fp32
    float* dx;
    float* dweight;   // [D] or null; needs rmsnorm_bwd_workspace_bytes of workspace
    void* workspace;
    long rows;
    int D;
    float eps;
};
hipError_t launch_rmsnorm_fwd(const RmsNormArgs& a, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const RmsNormArgs& a, hipStream_t s);
size_t rmsnorm_bwd_workspace_bytes(long rows, int D);
// The library's fixed device scratch for the backward's dweight partials on the current device
// (looked up once per device): its device address and size.
hipError_t rmsnorm_scratch(void** ptr, size_t* bytes);

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
    const int* cu_seqlens = nullptr;  // packed batch: B + 1 cumulative lengths (device), T = rows
};
// Single-kernel path (no workspace). Returns hipErrorNotSupported when it does not cover
// the arguments.
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t s);
bool chunk_supported(int T, int H, int DK, int DV, bool bf16);

// Sparse delta memory: product-key addressing of queries [queries = rows * H, dk] against per-head
// sub-key tables [H, n, dk/2] (two of them), giving m slots and weights per query; the
// token-by-token update of the slot memory M [B, H, N, dv] with its decay stamps [B, H, dv/64, N]
// and running log-decay sums L [B, H, dv/64] (fp64); and the fold of the stamps into M.
struct SdmAddressArgs {
    const void *x, *C1, *C2;
    long queries;
    int H, dk, n, m;
    bool bf16;
    int* idx;
    float* wt;
};
struct SdmFwdArgs {
    const void *v, *alpha, *b, *w;
    const int* widx;
    const float* wwt;
    const int* ridx;
    const float* rwt;
    float* M;
    double *stamp, *L;
    float* o;
    int B, T, H;
    long N;
    int dv, W, R;
    bool bf16;
};
bool sdm_address_supported(int dk, int n, int m);
bool sdm_fwd_supported(int dv, int W, int R);
hipError_t launch_sdm_address(const SdmAddressArgs& a, hipStream_t s);
hipError_t launch_sdm_fwd(const SdmFwdArgs& a, hipStream_t s);
hipError_t launch_sdm_fold(float* M, double* stamp, double* L, long heads, long N, int dv, hipStream_t s);

// Fused path (no workspace): one kernel per (b, h, 64-column tile) whose prep wavefronts build the
// next chunk's operands in LDS while its chain wavefronts run the current chunk. bf16, d_k = d_v in
// {64, 128}, every gate form and prologue flag.
hipError_t launch_fused(const ChunkArgs& a, hipStream_t s);
bool fused_supported(int T, int H, int DK, int DV, bool bf16);

// Two-kernel path (prep + chain) through a workspace ring of per-chunk operand blobs.
// Workspace = state buffer (B*H*DK*DV fp32) + R chunk slots of split_chunk_bytes each; with a
// slot for every chunk plus the segment buffers (split_workspace_bytes), a long sequence with few
// (b, h) runs its chain in parallel segments.
hipError_t launch_split(const ChunkArgs& a, hipStream_t s);
bool split_supported(int T, int H, int DK, int DV, bool bf16);
bool split_fwd_supported(int T, int H, int DK, int DV, bool bf16);  // also bf16 d = 256
bool varlen_fwd_supported(int T, int H, int DK, int DV, bool bf16);  // packed batches, forward
size_t split_chunk_bytes(int B, int H, int DK, bool bf16);
size_t split_workspace_bytes(int B, int T, int H, int DK, int DV, bool bf16);
// Two-kernel path over a packed batch of a.B sequences, a.T rows in all, delimited by
// a.cu_seqlens. Workspace (one round, no segments): the sequence table, then one slot per chunk
// of an upper bound on the chunk count (varlen_chunk_bound), per head.
hipError_t launch_split_varlen(const ChunkArgs& a, hipStream_t s);
long varlen_chunk_bound(int n, int T);
size_t varlen_table_bytes(int n);
size_t varlen_workspace_bytes(int n, int T, int H, int DK, int DV, bool bf16);
// The backward's forward pass over a packed batch (a.B sequences, a.T rows, a.cu_seqlens): the
// sequence table into `table` (varlen_table_bytes), the operand blocks into `blobs` ([h][chunk of
// the batch], `ring` = varlen_chunk_bound slots per head), the start state of every chunk
// ([h][chunk of the batch][DK][DV] fp32) and the rows of D' and Delta (fp16, packed rows). bf16
// inputs, general gates, the prologue flags allowed.
hipError_t launch_varlen_states(const ChunkArgs& a, char* table, char* blobs, long ring, uint16_t* S_save,
                                uint16_t* Dp_save, uint16_t* Dl_save, hipStream_t s);
// Prep over every chunk into `blobs` ([b*h][chunk] operand blocks), then the state-only chain in
// order, saving the state at the start of every chunk ([b*h][chunk][DK][DV]) and the rows of D'
// and Delta ([B, T, H, DV], fp16 bits). bf16 inputs, general gates, the prologue flags allowed.
hipError_t launch_split_states(const ChunkArgs& a, char* blobs, uint16_t* S_save, uint16_t* Dp_save, uint16_t* Dl_save,
                               hipStream_t s);

// Backward of the chunkwise prefill (bf16 inputs, general gates, d_k = d_v in {32, 64, 128}).
struct BwdArgs {
    const void *q, *k, *v, *alpha, *b, *w;
    const float *S0, *dO, *dS_T;
    float *dq, *dk, *dv, *dalpha, *db, *dw, *dS0;
    int B, T, H, DK, DV;
    bool bf16;
    uint32_t flags;
    void* workspace;
    size_t workspace_bytes;
    const int* cu_seqlens = nullptr;  // packed batch: B + 1 cumulative lengths (device), T = rows
    // the workspace already holds what launch_fwd_save left in it for these inputs: the operand
    // blocks, chunk-start states and D', Delta rows are read, not recomputed
    bool saved = false;
};
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s);
// The forward (o, S_T) that also leaves in a backward workspace (of bwd_workspace_bytes, or
// bwd_varlen_workspace_bytes for a packed batch) the operand blocks, the chunk-start states and
// the D', Delta rows (and, packed, the sequence table) that launch_bwd with `saved` reads.
hipError_t launch_fwd_save(const ChunkArgs& a, hipStream_t s);
bool bwd_supported(int T, int H, int DK, int DV, bool bf16, uint32_t flags);
size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV, uint32_t flags);
// The same for a packed batch of n sequences, T rows in all.
size_t bwd_varlen_workspace_bytes(int n, int T, int H, int DK, int DV, uint32_t flags);

}  // namespace gdn2
