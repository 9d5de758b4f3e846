/*
 * gdn2.h -- C ABI of the Gated DeltaNet-2 recurrence library for AMD Instinct MI355X (gfx950).
 *
 * Sources (pages, cited by title and paragraph):
 *   [GDN2-summary] "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами для раздельного
 *                  стирания и записи в линейном внимании" (edge.aivizor.me)
 *   [GDN2-news]    "NVIDIA улучшила память LLM без роста затрат на контекст" (arddev.tech)
 *
 * The operation. For every batch element b and head h independently, over tokens t = 1..T:
 *
 *     S_t = (I - k_t (b_t (.) k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T
 *     o_t = S_t^T q_t
 *
 * The update is [GDN2-summary, paragraph "Техническая схема", state-update equation]: alpha_t
 * is the channel-wise decay on the key axis, b_t in [0,1]^{d_k} the erase gate (key axis) and
 * w_t in [0,1]^{d_v} the write gate (value axis). The readout on the updated state is not
 * printed on the pages; it is the linear-attention reading of a history compressed into a
 * fixed state [GDN2-news, section "Контекст"]. No output scale is applied (pre-scale q).
 *
 * Scalar gates give the earlier models [GDN2-news, the authors' quote on special cases;
 * GDN2-summary, paragraph "Архитектурно"]: with one scalar beta_t per token, b_t = beta_t*1
 * and w_t = beta_t*1 (KDA when alpha stays channel-wise, Gated DeltaNet when alpha_t is a
 * scalar too). The flags below select these forms without materialising the gates.
 *
 * Layouts (row-major, contiguous, no padding):
 *   prefill  q, k, alpha, b : [B, T, H, d_k]     v, w, o : [B, T, H, d_v]
 *            scalar alpha   : [B, T, H]          scalar beta (passed as b) : [B, T, H]
 *   decode   q, k, alpha, b : [B, H, d_k]        v, w, o : [B, H, d_v]
 *            scalar alpha / beta : [B, H]
 *   state    S0, S_out, S   : [B, H, d_k, d_v] float32 (row i = key channel i)
 * Inputs q, k, v, alpha, b, w share one element type (in_dtype); o and the state are float32.
 *
 * Ownership and execution. All pointers are device pointers owned by the caller (HIP device
 * memory, e.g. allocated by PyTorch), the chunked prefill's optional workspace included. The
 * library allocates nothing, keeps no state between calls and is reentrant (two calls in
 * flight at once need two workspaces). Calls only enqueue kernels on `stream` (a hipStream_t;
 * NULL is the null stream) and return at once; inputs must stay alive and unchanged until the
 * stream passes the work.
 *
 * Errors. Argument errors are detected on the host and returned with nothing enqueued. A
 * failed launch returns GDN2_ERR_HIP. Device faults surface at the caller's next
 * synchronisation. Nothing is printed and nothing aborts.
 *
 * Preconditions not checked on the device: finite inputs; alpha in (0, 1] on the prefill
 * path (it takes log alpha); on the bf16 prefill paths, the per-chunk operands formed from q, k,
 * b and the decay below 6.5e4 (their matrix-core operands are fp16; see gdn2_chunk_fwd), and for
 * the backward also the state and its gradient below 6.5e4.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN2_ABI_VERSION 1

typedef enum {
    GDN2_OK = 0,
    GDN2_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN2_ERR_SHAPE = 2,       /* B <= 0, H <= 0, T < 0, or a size that overflows */
    GDN2_ERR_UNSUPPORTED = 3, /* (d_k, d_v), dtype or flags not supported */
    GDN2_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    GDN2_ERR_ALIAS = 5,       /* an output overlaps an input (other than S_out == S0) */
    GDN2_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    GDN2_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required */
    GDN2_ERR_SCRATCH = 8      /* the call needs more than the library's fixed scratch holds */
} gdn2_status;

typedef enum { GDN2_BF16 = 0, GDN2_F32 = 1 } gdn2_dtype;

enum {
    GDN2_ALPHA_SCALAR = 1u, /* alpha holds one decay per token, broadcast over d_k */
    GDN2_BETA_SCALAR = 2u,  /* b holds one beta per token: b = beta*1_{d_k}, w = beta*1_{d_v};
                               w must be NULL */
    /* Prologue flags: the steps in front of the recurrence done inside the kernels, in fp32, on
     * the inputs as given [GDN2-summary, paragraph "Архитектурно": L2-normalised q/k, sigmoid
     * gates]. Taken by the two-kernel and the fused prefill, the packed prefill, the
     * token-by-token prefill, the decode step and gdn2_chunk_bwd (which then gives the gradients
     * with respect to the raw inputs); the single-kernel prefill (no workspace, sizes the fused
     * kernel does not take) returns GDN2_ERR_UNSUPPORTED for them. */
    GDN2_QK_L2NORM = 4u,   /* q and k are normalised per token and head over d_k:
                              x / max(|x|_2, 1e-12) */
    GDN2_GATE_LOGITS = 8u  /* alpha, b, w (or the scalar forms) hold pre-activations x; the
                              gates are the logistic sigmoid 1 / (1 + e^-x), and log alpha is
                              taken directly as log sigma(x) */
};

/*
 * Chunkwise-parallel prefill. Runs the recurrence over T tokens from the initial state S0
 * (NULL = zeros), writes o for every token and the final state to S_out (NULL = not stored;
 * S_out == S0 is allowed, partial overlap is not). T == 0 copies S0 (or zeros) to S_out.
 *
 * The chunk length is 64 and the cumulative channel-wise decay is absorbed into the rank-1
 * factors of a WY/UT representation [GDN2-summary, paragraph "Реализация"]; the result equals
 * the token-by-token recurrence up to rounding. bf16 inputs use fp16 matrix-core operands with
 * fp32 accumulation and an fp32 state; fp32 inputs are computed in fp32 throughout.
 *
 * The workspace selects how the chunks are scheduled; the result is the same either way.
 *  - workspace != NULL with workspace_bytes > 0 (and the sizes supported below): two kernels. A
 *    prep kernel, parallel over every (b, h, chunk), computes each chunk's decay-scaled factors,
 *    its 64x64 Gram products and the UT inverse T, and stores them as one operand block per chunk
 *    in the workspace; a chain kernel then runs the state recurrence chunk by chunk from those
 *    blocks. The fastest schedule at every size it takes. Supported: bf16 with d in {32, 64, 128,
 *    256}, fp32 with d in {32, 64, 128}, any flags (the operand blocks of bf16 at d = 256 and of
 *    fp32 at d >= 64 are too large for two in the chain kernel's LDS: it keeps one and copies the
 *    next after each chunk; at fp32 d = 128 its chain wavefronts also load v and w straight into
 *    registers, for want of LDS room).
 *    Layout of the workspace: the fp32 state buffer [B, H, d_k, d_v]
 *    first when S_out is NULL (none when S_out is given), then R chunk slots of B*H operand
 *    blocks. R = (workspace_bytes - state bytes) / slot bytes chunks are prepared per round; with
 *    fewer slots than chunks the two kernels alternate over rounds of R chunks. When B*H is too
 *    small to fill the GPU and the sequence is long, a workspace of the size the query returns
 *    also holds per-segment buffers: the sequence is cut into segments whose state transitions
 *    are computed in parallel and combined by a scan, so the chain runs all segments at once (the
 *    result is the same recurrence, up to rounding). The buffer must be 256-byte aligned (else
 *    GDN2_ERR_ALIGN), hold the state and one slot (else GDN2_ERR_WORKSPACE) and overlap no input or
 *    output (else GDN2_ERR_ALIAS). Its contents are scratch on entry and on return.
 *  - no workspace (NULL or workspace_bytes == 0), bf16 with d in {64, 128}: the fused kernel, which
 *    allocates nothing and takes every gate form and prologue flag. One workgroup per (b, h,
 *    64-column tile of the state): four of its wavefronts run the state recurrence of chunk n while
 *    four others compute chunk n + 1's factors, Gram products and T into a second LDS buffer, so no
 *    operand goes through HBM (the algorithmic bytes only).
 *  - no workspace, other sizes: one kernel, one workgroup per (b, h, 64-column tile) computing
 *    each chunk's factors and then its part of the state recurrence. Supported: bf16 with d = 32,
 *    fp32 with d in {32, 64}; no prologue flags (GDN2_ERR_UNSUPPORTED).
 * Range: the bf16 paths round their products' operands to fp16. The state, and every per-chunk
 * product formed from it and from v, are held times a power of two chosen per wavefront and chunk
 * (exact), so the state may take any magnitude fp32 holds; the operands formed from q, k, b and the
 * decay (scaled q and k, the Gram blocks and T) must stay below 6.5e4, which holds for
 * L2-normalised q and k and gates in [0, 1].
 * d_k must equal d_v, else GDN2_ERR_UNSUPPORTED. A sequence may be of any length the grid and
 * the workspace allow: the kernels address each chunk's rows from a 64-bit base, so one call takes
 * sequences whose rows span more than 4 GiB (T >= 524,288 at H = 16, d = 128). Any flags above.
 */
gdn2_status gdn2_chunk_fwd(const void *q, const void *k, const void *v, const void *alpha,
                           const void *b, const void *w, const float *S0, float *o,
                           float *S_out, int32_t B, int32_t T, int32_t H, int32_t d_k,
                           int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for the two-kernel path of gdn2_chunk_fwd at these sizes: the state buffer
 * (when S_out may be NULL), one slot per chunk so that one round covers the sequence, and the
 * segment buffers when the sizes are segmented. 0 when the two-kernel path does not take these
 * sizes (pass NULL; the fused or the single kernel runs). */
size_t gdn2_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                      int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags);

/*
 * Prefill of N sequences of different lengths packed along the token axis, each run from its
 * own initial state exactly as gdn2_chunk_fwd runs one sequence (chunks of 64 counted from the
 * sequence's first token [GDN2-summary, paragraph "Реализация"]; no chunk spans two sequences).
 * The packing itself is a layout of this library, not of the method.
 *
 *   cu_seqlens  [N + 1] int32 in device memory: sequence s is rows cu_seqlens[s] ..
 *               cu_seqlens[s + 1] - 1. Expected: cu_seqlens[0] == 0, non-decreasing,
 *               cu_seqlens[N] == T_total (empty sequences allowed). The host does not read it; on
 *               the device each bound is clamped to [0, T_total] and the bounds are made
 *               non-decreasing, so other values cannot make the kernels touch memory outside the
 *               arrays, but rows then left outside every sequence keep their o unwritten.
 *   q, k, alpha, b  [T_total, H, d_k]; v, w [T_total, H, d_v] (scalar gates [T_total, H]);
 *               in_dtype, gate_flags and their layouts as in gdn2_chunk_fwd
 *   S0, S_out   [N, H, d_k, d_v] float32 (S0 NULL = zeros; S_out NULL = not stored;
 *               S_out == S0 allowed). A sequence without tokens gets S_out = S0.
 *   o           [T_total, H, d_v] float32
 *   workspace   required, 256-byte aligned, at least gdn2_chunk_fwd_varlen_workspace_bytes
 *               (the sequence table, then one operand block per chunk of
 *               (T_total + 63 N) / 64 chunks per head, which bounds the chunk count); scratch.
 *
 * Same two kernels as the workspace path of gdn2_chunk_fwd (one round, no segments), preceded by
 * a one-workgroup kernel that builds the sequence table. Supported sizes and errors as there:
 * bf16 and fp32 with d in {32, 64, 128}, d_k == d_v, any flags; GDN2_ERR_NULL without cu_seqlens, GDN2_ERR_WORKSPACE without a workspace or with
 * fewer bytes than the query returns, GDN2_ERR_ALIGN for a cu_seqlens not 4-byte aligned or a
 * workspace not 256-byte aligned, GDN2_ERR_ALIAS when an output or the workspace overlaps
 * anything else (S_out == S0 excepted), GDN2_ERR_SHAPE for N <= 0 or T_total < 0.
 */
gdn2_status gdn2_chunk_fwd_varlen(const void *q, const void *k, const void *v, const void *alpha,
                                  const void *b, const void *w, const float *S0, float *o,
                                  float *S_out, const int32_t *cu_seqlens, int32_t N,
                                  int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                  gdn2_dtype in_dtype, uint32_t gate_flags, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Workspace bytes for gdn2_chunk_fwd_varlen at these sizes; 0 when the sizes are not supported. */
size_t gdn2_chunk_fwd_varlen_workspace_bytes(int32_t N, int32_t T_total, int32_t H, int32_t d_k,
                                             int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags);

/*
 * Token-by-token prefill: the same result as gdn2_chunk_fwd, computed one token at a time in
 * fp32 (each state column tile stays in registers for the whole sequence). Same arguments,
 * layouts, errors and aliasing rules; no workspace. Supported: d_k, d_v in {32, 64, 128, 256}.
 */
gdn2_status gdn2_recurrent_fwd(const void *q, const void *k, const void *v, const void *alpha,
                               const void *b, const void *w, const float *S0, float *o,
                               float *S_out, int32_t B, int32_t T, int32_t H, int32_t d_k,
                               int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                               void *stream);

/*
 * One decode step for B*H independent sequences, constant memory per sequence (the state is
 * the whole history [GDN2-news, section "Контекст"]). Updates S in place,
 *     S <- (I - k (b (.) k)^T) Diag(alpha) S + k (w (.) v)^T,
 * and writes o = S^T q on the updated state. fp32 arithmetic; one read and one write of each
 * state. Supported: d_k, d_v in {32, 64, 128, 256}.
 */
gdn2_status gdn2_decode_step(const void *q, const void *k, const void *v, const void *alpha,
                             const void *b, const void *w, float *S, float *o, int32_t B,
                             int32_t H, int32_t d_k, int32_t d_v, gdn2_dtype in_dtype,
                             uint32_t gate_flags, void *stream);

/*
 * Backward of the prefill: the gradients of L = sum_t <dO_t, o_t> + <dS_T, S_T> for the recurrence
 * above (o_t and S_T as gdn2_chunk_fwd computes them from the same inputs), through the chunkwise
 * WY form with C = 64 [GDN2-summary, paragraph "Реализация"]. The forward is recomputed inside
 * the call; nothing from a previous gdn2_chunk_fwd call is needed.
 *
 *   inputs   q, k, v, alpha, b, w, S0 as in gdn2_chunk_fwd (S0 NULL = zeros);
 *            dO [B, T, H, d_v] float32 (required when T > 0);
 *            dS_T [B, H, d_k, d_v] float32 (NULL = zeros)
 *   outputs  dq, dk, dalpha, db [B, T, H, d_k] float32; dv, dw [B, T, H, d_v] float32;
 *            dS0 [B, H, d_k, d_v] float32 (NULL = not stored). Every output is overwritten.
 *   scalar gates (gate_flags GDN2_ALPHA_SCALAR, GDN2_BETA_SCALAR, the forms of gdn2_chunk_fwd):
 *            alpha [B, T, H] and dalpha [B, T, H] = dL/dalpha; beta passed as b [B, T, H] with
 *            w == NULL, and db [B, T, H] = dL/dbeta (the gradients through b and w summed), dw
 *            == NULL. A scalar gate is the general gate with the scalar in every channel, so its
 *            gradient is the sum of the per-channel gradients; the kernels read the scalars
 *            themselves and sum those gradients over the channels of each row.
 *
 *   prologue flags (GDN2_QK_L2NORM, GDN2_GATE_LOGITS): q, k, alpha, b, w are the raw inputs the
 *            forward takes with the same flags, and dq, dk, dalpha, db, dw are the gradients
 *            with respect to them (through the norm and the sigmoids).
 *
 * Supported: bf16 inputs, every gate form and prologue flag, d_k == d_v in {32, 64, 128}, and one
 * sequence's rows below 4 GiB ((T + 64)*H*d_v*4 < 2^32 bytes); anything else returns
 * GDN2_ERR_UNSUPPORTED. Arithmetic as in the forward: fp16 matrix-core operands with fp32
 * accumulation for the state chains and for the per-chunk products over the value channels (the
 * chunk-start states and chunk-end state gradients are kept in fp16, the precision those
 * products take them in), fp32 for the rest of the per-chunk gradient work.
 * The workspace (required when T > 0, 256-byte aligned, at least
 * gdn2_chunk_bwd_workspace_bytes for the same gate_flags) holds the operand blocks, the state and
 * its gradient at every chunk boundary and the per-chunk intermediate products (and, for scalar
 * gates, per token row the partial sums of their gradients over groups of channels, added up
 * by the call's last kernel; for the L2 norm, the row norms of q and k); its contents are
 * scratch. No output may
 * overlap an input, another output or the workspace (GDN2_ERR_ALIAS). Other errors, ownership
 * and stream semantics as for gdn2_chunk_fwd.
 */
gdn2_status gdn2_chunk_bwd(const void *q, const void *k, const void *v, const void *alpha,
                           const void *b, const void *w, const float *S0, const float *dO,
                           const float *dS_T, float *dq, float *dk, float *dv, float *dalpha,
                           float *db, float *dw, float *dS0, int32_t B, int32_t T, int32_t H,
                           int32_t d_k, int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes gdn2_chunk_bwd needs at these sizes; 0 when it does not take them (or T == 0,
 * which needs none). */
size_t gdn2_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                      gdn2_dtype in_dtype, uint32_t gate_flags);

/*
 * A training step's forward and backward without the recomputation: gdn2_chunk_fwd_save computes
 * o and S_T as gdn2_chunk_fwd does [GDN2-summary, paragraph "Реализация"] and, in the same pass,
 * leaves in a backward workspace what gdn2_chunk_bwd would otherwise recompute at its start (the
 * per-chunk operand blocks, the state at every chunk start and the D', Delta rows of every
 * chunk, all in the precision the backward takes them in); gdn2_chunk_bwd_saved then gives the
 * gradients gdn2_chunk_bwd gives, reading those instead of recomputing them.
 *
 *   gdn2_chunk_fwd_save: arguments as gdn2_chunk_fwd; the workspace is required when T > 0,
 *            256-byte aligned, at least gdn2_chunk_bwd_workspace_bytes for the same sizes and
 *            gate_flags, and overlaps no input or output (GDN2_ERR_ALIAS). Supported where
 *            gdn2_chunk_bwd is (bf16, d_k == d_v in {32, 64, 128}, every gate form and prologue
 *            flag); one sequence is one pass, never cut into segments. The state operands of the
 *            products are fp16 without the power-of-two rescaling gdn2_chunk_fwd applies (as in
 *            the backward's own recomputation), so the state's entries must stay inside fp16's
 *            range; o agrees with gdn2_chunk_fwd's to fp16 operand rounding.
 *   gdn2_chunk_bwd_saved: arguments and outputs as gdn2_chunk_bwd, with the workspace that a
 *            gdn2_chunk_fwd_save call on the same inputs, sizes and gate_flags filled, unchanged
 *            since (other calls may run in between). The call reads the saved parts and uses the
 *            rest as scratch, so it may be repeated on the same saves. Given any other
 *            workspace contents its gradients are undefined (no error can tell).
 */
gdn2_status gdn2_chunk_fwd_save(const void *q, const void *k, const void *v, const void *alpha,
                                const void *b, const void *w, const float *S0, float *o, float *S_out,
                                int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                gdn2_dtype in_dtype, uint32_t gate_flags, void *workspace,
                                size_t workspace_bytes, void *stream);
gdn2_status gdn2_chunk_bwd_saved(const void *q, const void *k, const void *v, const void *alpha,
                                 const void *b, const void *w, const float *S0, const float *dO,
                                 const float *dS_T, float *dq, float *dk, float *dv, float *dalpha,
                                 float *db, float *dw, float *dS0, int32_t B, int32_t T, int32_t H,
                                 int32_t d_k, int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags,
                                 void *workspace, size_t workspace_bytes, void *stream);
/* The same pair over a packed batch (the layouts, cu_seqlens and sizes of gdn2_chunk_fwd_varlen and
 * gdn2_chunk_bwd_varlen): gdn2_chunk_fwd_varlen_save takes a workspace of at least
 * gdn2_chunk_bwd_varlen_workspace_bytes (it also keeps the sequence table there) and
 * gdn2_chunk_bwd_varlen_saved reads it, with the same cu_seqlens contents. T_total == 0: the
 * forward writes S_out = S0 (or zeros) and needs no workspace. */
gdn2_status gdn2_chunk_fwd_varlen_save(const void *q, const void *k, const void *v, const void *alpha,
                                       const void *b, const void *w, const float *S0, float *o,
                                       float *S_out, const int32_t *cu_seqlens, int32_t N, int32_t T_total,
                                       int32_t H, int32_t d_k, int32_t d_v, gdn2_dtype in_dtype,
                                       uint32_t gate_flags, void *workspace, size_t workspace_bytes,
                                       void *stream);
gdn2_status gdn2_chunk_bwd_varlen_saved(const void *q, const void *k, const void *v, const void *alpha,
                                        const void *b, const void *w, const float *S0, const float *dO,
                                        const float *dS_T, float *dq, float *dk, float *dv, float *dalpha,
                                        float *db, float *dw, float *dS0, const int32_t *cu_seqlens,
                                        int32_t N, int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                        gdn2_dtype in_dtype, uint32_t gate_flags, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * Backward of gdn2_chunk_fwd_varlen: the gradients of L = sum over the packed rows of <dO, o> plus
 * sum over the sequences of <dS_T[s], S_T[s]>, for N sequences packed along the token axis and
 * delimited by cu_seqlens (device memory, read as by gdn2_chunk_fwd_varlen: clamped to
 * [0, T_total] and made non-decreasing). Each sequence is its own recurrence from S0[s], chunked
 * from its own first token [GDN2-summary, paragraph "Реализация"], so its gradients are those
 * gdn2_chunk_bwd gives for it alone.
 *
 *   inputs   q, k, alpha, b [T_total, H, d_k]; v, w [T_total, H, d_v] (scalar gates [T_total, H],
 *            w == NULL with GDN2_BETA_SCALAR); S0 [N, H, d_k, d_v] float32 (NULL = zeros);
 *            dO [T_total, H, d_v] float32; dS_T [N, H, d_k, d_v] float32 (NULL = zeros)
 *   outputs  dq, dk, dalpha, db [T_total, H, d_k] (scalar gates [T_total, H]); dv, dw
 *            [T_total, H, d_v]; dS0 [N, H, d_k, d_v] (NULL = not stored). Rows inside a sequence
 *            are overwritten; rows that bounds out of order leave outside every sequence are not
 *            written. A sequence without tokens gets dS0[s] = dS_T[s].
 *   workspace  required when T_total > 0, 256-byte aligned, at least
 *            gdn2_chunk_bwd_varlen_workspace_bytes: the sequence table and the blocks of
 *            gdn2_chunk_bwd for (T_total + 63 N) / 64 chunks per head, which bounds the chunk count.
 *
 * Gate forms, prologue flags, supported sizes (T_total in place of T), arithmetic and errors as
 * for gdn2_chunk_bwd; in addition GDN2_ERR_NULL without cu_seqlens and GDN2_ERR_ALIGN for a
 * cu_seqlens not 4-byte aligned.
 */
gdn2_status gdn2_chunk_bwd_varlen(const void *q, const void *k, const void *v, const void *alpha,
                                  const void *b, const void *w, const float *S0, const float *dO,
                                  const float *dS_T, float *dq, float *dk, float *dv, float *dalpha,
                                  float *db, float *dw, float *dS0, const int32_t *cu_seqlens,
                                  int32_t N, int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                  gdn2_dtype in_dtype, uint32_t gate_flags, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Workspace bytes gdn2_chunk_bwd_varlen needs at these sizes; 0 when it does not take them (or
 * T_total == 0, which needs none). */
size_t gdn2_chunk_bwd_varlen_workspace_bytes(int32_t N, int32_t T_total, int32_t H, int32_t d_k,
                                             int32_t d_v, gdn2_dtype in_dtype, uint32_t gate_flags);

/*
 * One decode step over a pool of states (serving: the batch rows name their sequences' slots).
 * Batch row b (inputs q, k, v, alpha, b, w and output o as in gdn2_decode_step, [B, H, d]) updates
 * S_pool[slots[b]] in place, S_pool being [n_slots, H, d_k, d_v] float32, and writes o[b]. slots
 * is a device array of B int32 (4-byte aligned). A row whose slot is negative or not below n_slots
 * is skipped: its o row and the pool are left as they are (padding rows). Two rows naming the
 * same slot in one call race (the result is unspecified). Same arithmetic, flags and head sizes as
 * gdn2_decode_step (the state-per-sequence constant decode memory of [GDN2-news, "Контекст"]).
 */
gdn2_status gdn2_decode_step_slots(const void *q, const void *k, const void *v, const void *alpha,
                                   const void *b, const void *w, float *S_pool, const int32_t *slots,
                                   float *o, int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                                   int32_t n_slots, gdn2_dtype in_dtype, uint32_t gate_flags,
                                   void *stream);

/*
 * Output RMS normalisation: the recurrent layer's output passes through an RMS norm
 * [GDN2-summary, paragraph "Архитектурно"]. Per row of d values (one head's d_v outputs of one
 * token; rows = B*T*H for a prefill's o, B*H for a decode step's):
 *     y = x / sqrt(mean(x^2) + eps) * weight
 *
 *   x       [rows, d] float32 (the o of any call above)
 *   weight  [d] float32, shared by the rows (NULL = ones)
 *   y       [rows, d], y_dtype GDN2_F32 or GDN2_BF16 (rounded to nearest even); y == x is
 *           allowed with GDN2_F32 (in place); any other overlap is GDN2_ERR_ALIAS
 *   eps     >= 0 and finite (GDN2_ERR_UNSUPPORTED otherwise); a zero row with eps == 0 gives
 *           NaN, as the formula does
 * Supported: d in {32, 64, 128, 256}; rows == 0 enqueues nothing. fp32 arithmetic, one read of x
 * and one write of y. Pointers 16-byte aligned. No workspace.
 */
gdn2_status gdn2_rmsnorm_fwd(const float *x, const float *weight, void *y, int64_t rows, int32_t d,
                             float eps, gdn2_dtype y_dtype, void *stream);

/*
 * Backward of gdn2_rmsnorm_fwd: given dy = dL/dy [rows, d] float32, writes dx = dL/dx [rows, d]
 * float32 and, when dweight != NULL, dweight = dL/dweight [d] (the sum over every row of
 * dy * x / sqrt(mean(x^2) + eps)). With s = (mean(x^2) + eps)^(-1/2), xh = x s and
 * u = dy * weight: dx = s (u - xh mean(xh u)) per row. dx == dy is allowed (in place); no other
 * overlap. dweight is summed in a fixed order (per-workgroup partials in the workspace, then one
 * pass over them), so it is the same from run to run. The workspace (needed only with dweight,
 * gdn2_rmsnorm_bwd_workspace_bytes, 16-byte aligned) is scratch. rows == 0 writes dweight = 0.
 */
gdn2_status gdn2_rmsnorm_bwd(const float *x, const float *weight, const float *dy, float *dx,
                             float *dweight, int64_t rows, int32_t d, float eps, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Workspace bytes gdn2_rmsnorm_bwd needs for dweight at these sizes (0: none, or unsupported). */
size_t gdn2_rmsnorm_bwd_workspace_bytes(int64_t rows, int32_t d);

/*
 * gdn2_rmsnorm_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same checks, kernels and results
 * (bit for bit), with the dweight partials in a fixed device array inside the library instead
 * of a caller workspace. The array holds 1 MiB (1024 partials of d <= 256 floats), which covers
 * every supported size; a call needing more would return GDN2_ERR_SCRATCH. Each GPU the library
 * runs on keeps its own copy until the process ends; its address is looked up on the first call
 * made with that device current. Nothing is allocated or freed and no workspace is taken. Calls
 * on one GPU share the array: two calls in flight at once on one GPU (on different streams, or
 * from different threads without ordering) race and give unspecified dweight. The array needs no
 * clearing between calls (every partial a call reads is written by that call).
 */
gdn2_status gdn2_rmsnorm_bwd_noalloc(const float *x, const float *weight, const float *dy, float *dx,
                                     float *dweight, int64_t rows, int32_t d, float eps, void *stream);

/* A static, human-readable name for a status code. */
const char *gdn2_status_str(gdn2_status s);

/* ---------------------------------------------------------------------------------------
 * Sparse delta memory (SDM) [SDM-news: aiweekly.co, "Meta FAIR dévoile SDM, un RNN linéaire à
 * mémoire sparse massive", second paragraph; SDM-review: gonzo_ML, "Sparse Delta Memory:
 * Scaling the State of Linear RNNs through Sparsity", TL;DR]: Gated DeltaNet with the dense
 * key-value outer product replaced by sparse writes and reads of a memory of N slots, each slot
 * holding d_v values; a product-key index picks W write and R read slots per token (W = R = 64
 * on the pages). The pages leave the update on the chosen slots open; these calls take the
 * Gated DeltaNet-2 update ["Техническая схема"] with the key replaced by the N-vector a_t of
 * write weights (zero off the W slots), per-token scalar decay alpha_t and erase b_t (they act
 * on the slot axis), the value-axis write gate w_t, and the read o_t = M_t^T r_t from the updated
 * memory with the read weights r_t:
 *     M_t = (I - b_t a_t a_t^T) alpha_t M_{t-1} + a_t (w_t * v_t)^T.
 * ------------------------------------------------------------------------------------- */

/* Product-key addressing. For each of rows*H queries x [rows, H, d_k] (bf16 or fp32, rows = B*T
 * tokens): the first and second half of x are scored against the head's sub-key tables
 * C1, C2 [H, n, d_k/2] (same dtype; exact products summed in fp32, in an order the matrix cores
 * fix, so near-equal scores may rank either way within that rounding); the m best sub-keys of
 * each half are kept and the m best of their pair sums give the slots i*n + j (of N = n*n) with
 * the softmax of the sums as weights, best first (equal scores or sums: lower index first).
 * Writes idx [rows, H, m] int32 and weight [rows, H, m] fp32. Use it with x = k for the write
 * addresses (m = W) and x = q for the read addresses (m = R).
 * Supported: d_k in {64, 128, 256}, n in {64, 128, 256, 512}, 1 <= m <= min(64, n). All pointers
 * 16-byte aligned device memory; outputs overlap no input. rows = 0 returns GDN2_OK. */
gdn2_status gdn2_sdm_address(const void *x, const void *C1, const void *C2, int64_t rows, int32_t H,
                             int32_t d_k, int32_t n, int32_t m, gdn2_dtype dtype, int32_t *idx,
                             float *weight, void *stream);

/* The SDM recurrence over T tokens of B sequences, one token after another.
 * v, w: [B, T, H, d_v] (w NULL: all ones); alpha, b: [B, T, H] scalars, all in dtype; alpha in
 * (0, 1] (alpha = 0 is taken as a decay of e^-1e6, which wipes the memory);
 * widx/wwt: [B, T, H, W] int32 slots / fp32 weights of the writes (distinct slots per token, as
 * gdn2_sdm_address gives; a slot outside [0, N) is skipped, as if its weight were 0); ridx/rwt:
 * [B, T, H, R] those of the reads.
 * The memory state, updated in place: M [B, H, N, d_v] fp32, and its decay bookkeeping, stamp
 * [B, H, d_v/64, N] and L [B, H, d_v/64] fp64. L is the running sum of log alpha; slot s holds
 * M[s] as of its last write and stamp[s] the L of that write, so its value now is
 * M[s] * exp(L - stamp[s]). A token therefore reads and writes only its W + R slots. Start from
 * M = M0 with stamp = 0 and L = 0; gdn2_sdm_fold brings every slot up to date (after it
 * M[s] is the memory itself). o: [B, T, H, d_v] fp32. Arithmetic fp32, the decay sums fp64.
 * Supported: d_v in {64, 128, 256}, 1 <= W, R <= 64 (and <= N), N <= 2^31 - 1. All pointers
 * 16-byte aligned; M, stamp, L and o overlap no input and each other. T = 0 or B = 0: GDN2_OK,
 * nothing changes. */
gdn2_status gdn2_sdm_fwd(const void *v, const void *alpha, const void *b, const void *w,
                         const int32_t *widx, const float *wwt, const int32_t *ridx, const float *rwt,
                         float *M, double *stamp, double *L, float *o, int32_t B, int32_t T, int32_t H,
                         int64_t N, int32_t d_v, int32_t W, int32_t R, gdn2_dtype dtype, void *stream);

/* Brings the memory of gdn2_sdm_fwd up to date: M[s] *= exp(L - stamp[s]) and stamp[s] = L for
 * every slot (shapes as there). */
gdn2_status gdn2_sdm_fold(float *M, double *stamp, double *L, int32_t B, int32_t H, int64_t N,
                          int32_t d_v, void *stream);

/* GDN2_ABI_VERSION of the built library. */
int gdn2_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN2_H */
