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
 * {0, 1}; scale any finite float, negative and zero included (callers
 * normally pass 1/sqrt(d); the pages fix no sign for it).  The kernels form
 * the scaled logits in fp32, so scale * <q, k> must stay within fp32 range.
 * B, H, N >= 0; a call with B*H*N == 0 does nothing and returns ATTN_OK (the
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
#include <stdint.h>

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
    ATTN_E_HIP = 7,         /* the HIP runtime reported an error at launch */
    ATTN_E_TOO_LARGE = 8    /* attn_bwd_noalloc: B*H*N exceeds ATTN_NOALLOC_MAX_ROWS */
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
 * problem): the fp32 row terms -D_i (D_i = <dO_i, O_i>), [B, H, N], rounded up to a
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

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  The D terms live in a fixed 4 MiB device array of
 * the library instead of the caller's workspace: each GPU the library runs on
 * holds one copy of it until the process ends.  The call itself allocates
 * nothing.  Arguments, layout, results and errors are those of attn_bwd
 * (results are bitwise equal to attn_bwd's), except:
 *   - B*H*N must not exceed ATTN_NOALLOC_MAX_ROWS (1048576 query rows);
 *     larger problems return ATTN_E_TOO_LARGE and enqueue nothing;
 *   - every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that
 *     overlap on one GPU -- on different streams, or from different threads
 *     without ordering -- race on it and give wrong gradients; callers must
 *     serialise them (one stream, or events between streams);
 *   - the first call on a device looks up the array's device address
 *     (hipGetSymbolAddress); a failure there returns ATTN_E_HIP.
 */
#define ATTN_NOALLOC_MAX_ROWS 1048576
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * Block-sparse attention: the tile skipping of all-zero mask blocks that the
 * snabindia page describes (chapter 1 and section 3.1), with the mask given
 * explicitly.  The key and query sequences are cut into blocks of
 * ATTN_MASK_BLOCK = 128 positions; key j is visible from query i only if
 * block_mask[m][i / 128][j / 128] != 0 (and, with causal = 1, j <= i).  Pairs
 * of blocks whose byte is 0 are never loaded or computed; the result is exact
 * attention under that mask.  A query row that sees no key gets O = 0 and
 * lse = -inf (and dQ = 0).
 *   block_mask : device bytes [mask_heads, nb, nb], nb = ceil(N / 128),
 *                row-major, owned by the caller, read-only (no alignment
 *                requirement); must not overlap any output.
 *   mask_heads : 1 (one mask for every batch and head), H (one per head,
 *                shared by the batches) or B*H (one per batch and head:
 *                m = b*H + h); anything else returns ATTN_E_SHAPE.
 * All other arguments, layouts and errors are those of attn_fwd / attn_bwd;
 * a NULL block_mask with B*H*N > 0 returns ATTN_E_NULL.  The backward takes
 * the same mask as the forward whose o and lse it is given, and the same
 * workspace as attn_bwd (attn_bwd_workspace_bytes).
 */
#define ATTN_MASK_BLOCK 128

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int N, int d, const uint8_t* block_mask, int mask_heads,
                         int causal, float scale, int dtype, void* stream);

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, const uint8_t* block_mask, int mask_heads,
                         int causal, float scale, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length batches, rectangular shapes and sliding windows.
 *
 * Layout.  A call holds `batch` independent sequences packed along the row
 * axis: q, o are [H, total_q, d], k, v are [H, total_k, d], lse is
 * [H, total_q] fp32.  Sequence b owns query rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of
 * every head.  cu_seqlens_q and cu_seqlens_k are DEVICE arrays of batch+1
 * int32 offsets (0 first, non-decreasing, total last); the kernels clamp every
 * offset to [0, total] and treat a decreasing pair as an empty sequence, so
 * bad offsets give wrong rows but never an out-of-bounds access.  This is the
 * padding-free form of the variable-length masking the yunthe article's
 * section 三.3 describes: no [B,1,N,N] mask is ever built.
 *
 * Rectangular sequences.  A sequence may have nq != nk; its query rows are
 * aligned to the end of its keys: row i sits at key position
 * pos = i + nk - nq (the prefill-with-cache shape).
 *
 * Visible keys.  Key j is visible to row i iff (causal == 0 or j <= pos) and
 * (window_left < 0 or j >= pos - window_left) and (window_right < 0 or
 * j <= pos + window_right): a sliding local window of the kind the yunthe
 * article's hybrid local/global attention uses (section 三.1), applied
 * exactly; key tiles outside every row's window are skipped, tiles inside
 * every row's window run unmasked.  A row that sees no key gets O = 0 and
 * lse = -inf.  window_left, window_right >= -1 (-1: unbounded); a window of
 * total_q + total_k or more reaches every key and is taken as unbounded.
 * total_q + total_k must not exceed 2^30 (ATTN_E_SHAPE otherwise), so that
 * every position and window bound fits a 32-bit integer on the device.
 *
 * max_seqlen_q (and max_seqlen_k for the backward) bound the grid: rows of a
 * longer sequence past that length are not computed and their outputs are
 * left unwritten.  Other arguments, memory, errors: as for attn_fwd /
 * attn_bwd (empty calls -- batch*H == 0, total_q == 0 or max_seqlen_q == 0
 * for the forward -- return ATTN_OK without examining pointers).
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int H,
                    int total_q, int total_k, int max_seqlen_q, int d, int causal,
                    int window_left, int window_right, float scale, int dtype, void* stream);

/* Workspace bytes of attn_bwd_varlen: one fp32 per query row (H * total_q),
 * rounded up to 256; (size_t)-1 for negative sizes. */
size_t attn_bwd_varlen_workspace_bytes(int H, int total_q);

/*
 * Backward of attn_fwd_varlen by recomputation.  dq is [H, total_q, d]; dk,
 * dv are [H, total_k, d]; o and lse come from attn_fwd_varlen with the same
 * arguments.  Keys that no query row sees get zero gradients.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int H,
                    int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                    int window_left, int window_right, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The standard, unfused forward -- a measurement baseline, not a fast path.
 * It runs the three passes of the hotdry blog's section on the memory
 * bandwidth bottleneck of traditional attention as three kernels with their
 * intermediates in device memory: S = scale Q K^T (fp32 [B, H, N, N], the
 * full matrix even when causal), P = softmax(S) (16-bit [B, H, N, N], causal
 * entries zero) with lse, then O = P V.  Arguments and outputs as attn_fwd;
 * `workspace` (16-byte aligned, caller-owned) holds S and P:
 * attn_fwd_unfused_workspace_bytes(B, H, N) bytes, about 6 N^2 bytes per
 * head.  B*H <= 65535 and N <= 2^24.  Compared with attn_fwd it shows the
 * O(N^2) device-memory traffic the fused kernel avoids.
 */
size_t attn_fwd_unfused_workspace_bytes(int B, int H, int N);
int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, int causal, float scale, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* A static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_EXACT_ATTN_H */
