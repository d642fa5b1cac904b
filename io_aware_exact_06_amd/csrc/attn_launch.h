// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and
// the kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kDtypeF16 = 0;
constexpr int kDtypeBF16 = 1;

// Where the sequences of a call live and which keys each query row sees.
//
// Dense calls (mode 0): tensors [B, H, N, d]; sequence s = b*H + h owns rows
// s*N .. s*N+N-1 of both the query and the key arrays.
// Packed calls (mode 1): tensors [H, total, d]; sequence s = h*B + b (B is the
// number of sequences) owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
// cu_k[b] .. cu_k[b+1]-1 of head h (cu_* are device int32 arrays, clamped to
// [0, total] and made non-decreasing on the device before use).
//
// Query row i of a sequence with nq rows and nk keys sits at key position
// pos = i + nk - nq (rows aligned to the end of the keys).  Key j is visible
// iff (wl < 0 or j >= pos - wl) and (wr < 0 or j <= pos + wr); a causal call
// is wr = 0.
//
// Block mask (dense calls only; bmask == nullptr: none): bytes
// [bm_heads, bm_nb, bm_nb], bm_nb = ceil(N / kMaskBlock); key j is visible
// from row i of sequence s = b*H + h only if bmask[m][i / 128][j / 128] != 0
// with m = 0 (bm_heads == 1), h (bm_heads == H) or s (bm_heads == B*H).
constexpr int kMaskBlock = 128;

struct SeqLayout {
    int mode;
    int B, H, N;
    const int* cu_q;
    const int* cu_k;
    int total_q, total_k;
    int wl, wr;
    const uint8_t* bmask;
    int bm_heads, bm_nb;
};

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    SeqLayout L;
    int max_nq;  // longest query sequence (grid size)
    int d, dtype;
    float scale;
    void* stream;
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;  // fp32 row terms D_i = <dO_i, O_i>, one per query row: the caller's workspace
    SeqLayout L;
    int max_nq, max_nk;  // longest query / key sequences (grid sizes)
    int d, dtype;
    float scale;
    void* stream;
};

// Bytes of backward workspace for `rows` query rows: one fp32 D per row,
// rounded up to a multiple of 256.
inline size_t bwd_workspace_bytes_rows(int64_t rows) {
    return (((size_t)rows * sizeof(float)) + 255) & ~(size_t)255;
}

// The unfused three-pass baseline (S and P in the caller's workspace).
struct UnfusedParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    void* workspace;
    int B, H, N, d, causal, dtype;
    float scale;
    void* stream;
};

// Workspace of the unfused baseline: fp32 S [BH, N, N], then 16-bit P [BH, N, N],
// each region rounded up to 256 bytes.
inline size_t unfused_score_bytes(int64_t B, int64_t H, int64_t N) {
    return (((size_t)(B * H * N) * (size_t)N * 4) + 255) & ~(size_t)255;
}
inline size_t unfused_workspace_bytes(int64_t B, int64_t H, int64_t N) {
    return unfused_score_bytes(B, H, N) + ((((size_t)(B * H * N) * (size_t)N * 2) + 255) & ~(size_t)255);
}

// Fixed device scratch of attn_bwd_noalloc (attn_noalloc.hip): room for the
// per-row D terms of B*H*N <= kScratchBytes / 4 query rows.
constexpr size_t kScratchBytes = (size_t)4 << 20;

// Device address of that scratch on the device that `stream` belongs to
// (looked up once per device, thread-safe).
hipError_t scratch_for_stream(void* stream, void** ptr);

hipError_t launch_fwd(const FwdParams& p);
hipError_t launch_unfused(const UnfusedParams& p);
hipError_t launch_bwd(const BwdParams& p);

}  // namespace attn
