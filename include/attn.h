/*
 * attn.h -- C ABI of a fused exact-attention library for one AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is the exact attention of the pages this library follows:
 *
 *     O = softmax(scale * Q K^T  [+ causal mask]) V
 *
 * computed block by block with an online softmax (running row maximum and
 * row sum, rescaling the partial output whenever the maximum grows), never
 * writing the score or probability matrices to device memory, and storing
 * only O and one fp32 statistic per query row.  The backward pass recomputes
 * the score blocks from that statistic (blog "Gemini 3 Flash的注意力内核重写：
 * 算子融合如何实现亚毫秒级推理", sections "1. 内核融合策略", "3. 在线softmax算法"
 * and "4. 重计算（Recomputation）策略"; the causal variant skips the upper
 * triangle as in the flash_attn_func(..., causal=True) example of chapter 1 of
 * the snabindia page on FlashAttention-3).
 *
 * Layout.  Q, K, V, O, dO, dQ, dK, dV are contiguous row-major tensors
 * [B, H, N, d] of 16-bit floats (the [B, H, T, D] layout of the snabindia
 * page, section 2.3); lse is a contiguous fp32 [B, H, N].  Query and key
 * sequences have the same length N.  With causal = 1, query i sees keys
 * j <= i.  lse[b,h,i] = ln sum_j exp(scale * <q_i, k_j>) over the visible keys
 * (natural logarithm of the scaled logits).
 *
 * Supported values.  d in {64, 128}; dtype ATTN_F16 or ATTN_BF16; causal in
 * {0, 1}; scale finite and >= 0 (callers normally pass 1/sqrt(d)).  B, H,
 * N >= 0; a call with B*H*N == 0 does nothing and returns ATTN_OK (the
 * pointers are then not examined).  Any N >= 1 works, including lengths that
 * are not a multiple of the kernels' tiles.
 *
 * Memory and ownership.  Every pointer is a device pointer owned by the
 * caller; the library allocates nothing and keeps no pointer after it
 * returns.  Tensor pointers must be 16-byte aligned, lse 4-byte aligned.  No
 * output may overlap an input or another output (inputs may alias each
 * other).  Work is enqueued on `stream` (a hipStream_t; NULL means the null
 * stream) and the call returns without waiting: buffers must stay alive until
 * the stream has executed the work.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; a
 * rejected call returns a nonzero status and has no side effect.  A failed
 * kernel launch returns ATTN_E_HIP.  Faults during execution surface at the
 * caller's next synchronisation, as for any HIP work.  The functions are
 * reentrant.  Both passes are bitwise deterministic (no atomics).
 */
#ifndef IO_AWARE_EXACT_ATTN_H
#define IO_AWARE_EXACT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype { ATTN_F16 = 0, ATTN_BF16 = 1 };

enum attn_status {
    ATTN_OK = 0,
    ATTN_E_NULL = 1,        /* a required pointer is NULL */
    ATTN_E_SHAPE = 2,       /* negative size, or sizes whose byte counts overflow */
    ATTN_E_UNSUPPORTED = 3, /* d, dtype, causal or scale outside the supported values */
    ATTN_E_ALIGN = 4,       /* a pointer is not aligned as required */
    ATTN_E_ALIAS = 5,       /* an output overlaps an input or another output */
    ATTN_E_WORKSPACE = 6,   /* backward workspace missing or smaller than required */
    ATTN_E_HIP = 7          /* the HIP runtime reported an error at launch */
};

/*
 * Forward pass.
 *   q, k, v : [B, H, N, d] inputs in `dtype`.
 *   o       : [B, H, N, d] output in `dtype`, O = softmax(scale Q K^T) V row by row.
 *   lse     : [B, H, N] fp32 output, the per-row logsumexp defined above.
 * Returns an attn_status.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for these sizes (0 for an empty
 * problem): the fp32 row terms D_i = <dO_i, O_i>, [B, H, N], rounded up to a
 * multiple of 256 bytes.  Returns (size_t)-1 for negative sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass by recomputation (blog section 4 above): the score blocks are
 * rebuilt from q, k and lse, so no N x N matrix is stored.
 *   q, k, v, o, dout : [B, H, N, d] in `dtype` (o and lse from attn_fwd with
 *                      the same arguments; dout is dL/dO).
 *   lse              : [B, H, N] fp32.
 *   dq, dk, dv       : [B, H, N, d] outputs in `dtype`.
 *   workspace        : device buffer of at least attn_bwd_workspace_bytes()
 *                      bytes, 16-byte aligned, owned by the caller; its
 *                      contents on entry do not matter and on return are
 *                      unspecified.  It must not overlap any other argument.
 * Gradients follow dV = P^T dO, dS = P o (dO V^T - D), dQ = scale dS K,
 * dK = scale dS^T Q with P = exp(scale Q K^T - lse) and D_i = <dO_i, O_i>.
 * Returns an attn_status.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int H, int N, int d, int causal, float scale, int dtype,
             void* workspace, size_t workspace_bytes, void* stream);

/* A static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_EXACT_ATTN_H */
