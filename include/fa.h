/*
 * fa.h — C ABI of the exact tiled attention library for MI355X (gfx950).
 *
 * The operation is exact attention, O = softmax(scale * Q K^T) V, per
 * (batch, head) slice, as defined in "Flash attention and efficient attention
 * — Hinglish notes", section "The Standard Attention Problem" (scores, row
 * softmax, weighted sum of values). The forward pass streams K/V tiles
 * through on-chip memory and merges per-tile row maximum m and row sum l with
 * the rescaling rule of that page's "Derivation: Incremental Softmax"
 * (Steps 2–3), so the N x N score matrix never reaches device memory. The
 * backward pass recomputes scores and probabilities on chip from Q, K and the
 * saved log-sum-exp, as the same page's "Backward Pass: Recomputation" says.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, contiguous, row-major [B][H][N][d] (d fastest);
 *    LSE is [B][H][N] float32. All pointers are DEVICE pointers of the
 *    current HIP device, 16-byte aligned.
 *  - dtype FA_BF16: bfloat16 storage, products accumulated in float32,
 *    d in {64, 128}. dtype FA_F32: float32 storage and arithmetic,
 *    1 <= d <= 128.
 *  - scale: any finite float (0 and negative values are allowed).
 *  - mask: FA_MASK_NONE; FA_MASK_CAUSAL (key j allowed iff j <= query i,
 *    square, top-left aligned); FA_MASK_LOCAL (allowed iff |i - j| <= window,
 *    the symmetric band of the notes' "Worked example Local Attention
 *    Window", whose 6 x 6 matrix is window = 1). window is ignored unless
 *    mask == FA_MASK_LOCAL and must then be >= 0. Every query row keeps at
 *    least its own key, so no row is empty.
 *  - Ownership: the caller owns and allocates every buffer; the library
 *    keeps no pointer after a call returns and allocates no device memory.
 *  - Outputs are fully overwritten and must not overlap any input.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL means the
 *    default stream) and the call returns without synchronizing. Argument
 *    errors are reported before anything is enqueued; a launch failure is
 *    reported as FA_ERR_LAUNCH; faults during execution surface at the
 *    caller's next synchronization.
 *  - Limits: B, H, N >= 1; B*H <= 2^31-1; N <= 2^29; N*d <= 2^31-1.
 *    Any window >= N - 1 allows every pair of a sequence (the band then
 *    equals no mask); windows up to 2^31 - 1 are accepted.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,     /* B, H or N < 1, or a size limit exceeded */
    FA_ERR_DTYPE = 3,     /* unknown dtype */
    FA_ERR_HEADDIM = 4,   /* d not supported for this dtype */
    FA_ERR_MASK = 5,      /* unknown mask, or window < 0 with FA_MASK_LOCAL */
    FA_ERR_SCALE = 6,     /* scale is NaN or infinite */
    FA_ERR_ALIGN = 7,     /* a pointer is not 16-byte aligned */
    FA_ERR_WORKSPACE = 8, /* workspace missing or smaller than required */
    FA_ERR_LAUNCH = 9,    /* the HIP runtime rejected a kernel launch */
    FA_ERR_ALIAS = 10,    /* an output buffer overlaps an input buffer */
    FA_ERR_CONFIG = 11    /* unknown kernel configuration (fa_tuning.h only) */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_LOCAL = 2 } fa_mask;

/*
 * Forward pass.
 *   q, k, v : inputs [B][H][N][d] in `dtype`.
 *   o       : output [B][H][N][d] in `dtype`: O_i = sum_j P_ij v_j with
 *             P_ij = exp(z_ij - LSE_i) over allowed j, z_ij = scale <q_i, k_j>.
 *   lse     : output [B][H][N] float32: LSE_i = m_i + ln l_i in natural-log
 *             units of the scaled, masked logits (m_i the row maximum, l_i the
 *             row sum of exp(z_ij - m_i)); the backward pass consumes it.
 * With FA_BF16 the weights are rounded to bfloat16 before they multiply V,
 * and each output row is divided by the float32 sum of those rounded
 * weights, so that it is a convex combination of value rows up to float32
 * rounding; LSE keeps the sum of the unrounded weights.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, fa_dtype dtype,
                 float scale, fa_mask mask, int window, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem: one float32 per
 * query row (D_i = <dO_i, O_i>), rounded up to 256 bytes. Returns 0 for an
 * invalid problem description.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Backward pass of the forward above for the loss whose gradient w.r.t. O is
 * dout. Recomputes P_ij = exp(z_ij - LSE_i) on chip (nothing N x N is read or
 * written) and returns
 *   dV_j = sum_i P_ij dO_i,
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *   with dS_ij = P_ij (<dO_i, v_j> - D_i) and D_i = <dO_i, O_i>.
 *   q, k, v, o, dout : inputs [B][H][N][d] in `dtype` (o and lse as written
 *                      by fa_fwd with the same scale and mask).
 *   lse              : input [B][H][N] float32.
 *   dq, dk, dv       : outputs [B][H][N][d] in `dtype`.
 *   workspace        : device buffer of at least
 *                      fa_bwd_workspace_bytes(...) bytes, owned by the caller,
 *                      contents ignored on entry and undefined on return.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int N, int d, fa_dtype dtype,
                 float scale, fa_mask mask, int window, void* stream);

/*
 * Backward pass without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory at call time: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc. Same operation, arguments, results and errors as fa_bwd, minus
 * the workspace: D_i = <dO_i, O_i> goes to a static device array of
 * FA_BWD_NOALLOC_MAX_ROWS floats (64 MiB) that the library holds on every GPU
 * it runs on until the process ends.
 *   B * H * N must not exceed FA_BWD_NOALLOC_MAX_ROWS (else FA_ERR_WORKSPACE,
 *   before anything is enqueued).
 *   Every call on one GPU shares that GPU's array: calls that can overlap on
 *   one GPU (different streams, or different host threads without ordering)
 *   race and may return wrong gradients; calls ordered on one stream are safe.
 *   The first call on a device looks up the array's address on that device
 *   (no allocation); FA_ERR_LAUNCH if that fails.
 */
#define FA_BWD_NOALLOC_MAX_ROWS (1u << 24)
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, fa_dtype dtype,
                         float scale, fa_mask mask, int window, void* stream);

/*
 * Bytes of device workspace fa_fwd_standard needs: the scores S (float32,
 * B*H*N rows of N rounded up to 4) and the probabilities P (bf16, rows of N
 * rounded up to 8), each region rounded up to 256 bytes. O(B*H*N^2): at
 * [1,16,16384,*] this is 25.8 GB. Returns 0 for an invalid problem or a
 * dtype other than FA_BF16.
 */
size_t fa_fwd_standard_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Standard (unfused) attention, the baseline fa_fwd is measured against: the
 * three steps of the notes' "The Standard Attention Problem" (scores
 * S = scale Q K^T, row softmax P, O = P V), each making a round trip through
 * device memory, which is the traffic the notes' "Memory Hierarchy" section
 * counts. Same O and LSE contract as fa_fwd. Every (query, key) pair is
 * computed; masked pairs get score -inf and probability 0. P is normalized
 * before it is rounded to bf16 and multiplied by V; each output row is then
 * divided by its row sum of the rounded P (1 up to that rounding).
 *   q, k, v, o, lse : as fa_fwd; dtype must be FA_BF16 (d in {64, 128}).
 *   workspace       : device buffer of at least
 *                     fa_fwd_standard_workspace_bytes(...) bytes, owned by the
 *                     caller, 16-byte aligned, not overlapping any tensor;
 *                     contents ignored on entry and undefined on return.
 * Errors: as fa_fwd; FA_ERR_DTYPE for FA_F32; FA_ERR_WORKSPACE when the
 * workspace is missing or too small; FA_ERR_SHAPE when B*H*N > 2^31-1.
 */
fa_status fa_fwd_standard(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int B, int H, int N, int d, fa_dtype dtype,
                          float scale, fa_mask mask, int window, void* stream);

/*
 * Bytes of device workspace fa_bwd_standard needs for its own intermediates:
 * dP (float32) and dS (bf16), in the layout of fa_fwd_standard's workspace,
 * so the same number of bytes. Returns 0 as fa_fwd_standard_workspace_bytes.
 */
size_t fa_bwd_standard_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Standard (unfused) backward, the baseline fa_bwd is measured against: it
 * reads the probabilities P that fa_fwd_standard stored instead of
 * recomputing them (the contrast the notes' "Backward Pass: Recomputation"
 * draws), and every N x N intermediate makes a round trip through device
 * memory: dP = dO V^T (float32), dV = P^T dO, D_i = sum_j P_ij dP_ij and
 * dS = P (dP - D) (bf16), dQ = scale dS K, dK = scale dS^T Q. Same gradients
 * as fa_bwd (up to rounding); masked pairs need no mask here, as their P is 0.
 *   q, k, v, dout  : inputs [B][H][N][d], bf16 (d in {64, 128}).
 *   fwd_workspace  : the workspace of a fa_fwd_standard call with the same
 *                    q, k, v, scale and mask, at least
 *                    fa_fwd_standard_workspace_bytes(...) bytes; read only.
 *   dq, dk, dv     : outputs [B][H][N][d] bf16.
 *   workspace      : at least fa_bwd_standard_workspace_bytes(...) bytes,
 *                    owned by the caller, 16-byte aligned, overlapping no
 *                    other buffer; contents ignored and undefined on return.
 * Errors: as fa_bwd; FA_ERR_DTYPE for FA_F32; FA_ERR_WORKSPACE when either
 * workspace is missing or too small; FA_ERR_SHAPE when B*H*N > 2^31-1.
 */
fa_status fa_bwd_standard(const void* q, const void* k, const void* v, const void* dout,
                          const void* fwd_workspace, size_t fwd_workspace_bytes,
                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                          int B, int H, int N, int d, fa_dtype dtype, float scale, void* stream);

/*
 * Bytes of device workspace fa_fwd_keymajor needs: the running state of
 * every query row (float32 unnormalized output, maximum, denominator and the
 * sum of the bf16-rounded weights, held by two lanes per row),
 * B*H*ceil(N/256)*512*(d/2 + 3)*4 bytes.
 * Returns 0 for an invalid problem or
 * a dtype other than FA_BF16.
 */
size_t fa_fwd_keymajor_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Key-major forward, the loop order of the FlashAttention paper's
 * Algorithm 1 as quoted in "What the tiling is actually constrained by"
 * (section "The formula, which the title only gestures at": K and V split
 * into T_c = ceil(N / B_c) blocks of B_c keys, block_keys here) and named in
 * the TensorViz card's fidelity note. The outer loop runs over key blocks
 * (one launch each); every launch updates the running state of all query
 * rows with the rule of the Hinglish notes' "Derivation: Incremental
 * Softmax" (Steps 2-3), reading the state from `workspace` and writing it
 * back, so its device-memory traffic grows as N^2 d / B_c. Same O and LSE
 * contract as fa_fwd (bf16 only), for comparison with fa_fwd's query-major
 * order.
 *   block_keys : 32, 64 or 128; also 256 when d == 64.
 *   workspace  : at least fa_fwd_keymajor_workspace_bytes(...) bytes, owned
 *                by the caller, 16-byte aligned, not overlapping any tensor;
 *                contents ignored on entry and undefined on return.
 * Errors: as fa_fwd; FA_ERR_DTYPE for FA_F32; FA_ERR_SHAPE for an
 * unsupported block_keys; FA_ERR_WORKSPACE.
 */
fa_status fa_fwd_keymajor(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int B, int H, int N, int d, fa_dtype dtype,
                          float scale, fa_mask mask, int window, int block_keys, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
