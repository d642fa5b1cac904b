// attn_api.cpp -- the C ABI declared in include/attn.h: host-side argument
// checks (all of them before anything is enqueued), then dispatch to the
// kernel launchers.
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include "attn_launch.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

Range range_of(const void* p, size_t bytes) {
    const uintptr_t u = (uintptr_t)p;
    return Range{u, u + bytes};
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared checks of sizes and scalar arguments.  On success *elems holds
// B*H*N*d and *rows B*H*N.
int check_common(int B, int H, int N, int d, int causal, float scale, int dtype, int64_t* rows,
                 int64_t* elems) {
    if (B < 0 || H < 0 || N < 0 || d < 0) return ATTN_E_SHAPE;
    if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_E_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_E_UNSUPPORTED;
    const int64_t bh = (int64_t)B * H;  // < 2^62
    // Every byte count below (B*H*N*d*4 at most, d <= 128) must fit in int64.
    if (bh != 0 && (int64_t)N > INT64_MAX / 512 / bh) return ATTN_E_SHAPE;
    const int64_t r = bh * N;
    *rows = r;
    *elems = r * d;
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_E_NULL: return "a required pointer is NULL";
        case ATTN_E_SHAPE: return "negative size, or sizes whose byte counts overflow";
        case ATTN_E_UNSUPPORTED: return "unsupported d, dtype, causal flag or scale";
        case ATTN_E_ALIGN: return "a pointer is not aligned as required";
        case ATTN_E_ALIAS: return "an output overlaps an input or another output";
        case ATTN_E_WORKSPACE: return "backward workspace missing or too small";
        case ATTN_E_HIP: return "the HIP runtime reported an error at launch";
        case ATTN_E_TOO_LARGE: return "the problem exceeds the fixed scratch of the allocation-free entry point";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Bytes of a block mask [mask_heads, nb, nb], nb = ceil(N / 128); 0 when the
// call's mask_heads is not 1, H or B*H.
size_t mask_bytes(int B, int H, int N, int mask_heads) {
    const int64_t bh = (int64_t)B * H;
    if (mask_heads != 1 && mask_heads != H && mask_heads != bh) return 0;
    if (mask_heads <= 0) return 0;
    const int64_t nb = ((int64_t)N + attn::kMaskBlock - 1) / attn::kMaskBlock;
    return (size_t)mask_heads * (size_t)nb * (size_t)nb;
}

attn::SeqLayout dense_layout(int B, int H, int N, int causal, const uint8_t* bm, int mask_heads) {
    attn::SeqLayout L{0, B, H, N, nullptr, nullptr, N, N, -1, causal ? 0 : -1, bm, mask_heads,
                      (N + attn::kMaskBlock - 1) / attn::kMaskBlock};
    return L;
}

int fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
              const uint8_t* bm, int mask_heads, int causal, float scale, int dtype, void* stream) {
    int64_t rows = 0, elems = 0;
    int st = check_common(B, H, N, d, causal, scale, dtype, &rows, &elems);
    if (st != ATTN_OK) return st;
    if (rows == 0) return ATTN_OK;
    size_t mb = 0;
    if (bm) {
        mb = mask_bytes(B, H, N, mask_heads);
        if (mb == 0) return ATTN_E_SHAPE;
    }
    if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return ATTN_E_ALIGN;
    const size_t tb = (size_t)elems * 2, lb = (size_t)rows * 4;
    const Range rq = range_of(q, tb), rk = range_of(k, tb), rv = range_of(v, tb);
    const Range ro = range_of(o, tb), rl = range_of(lse, lb);
    if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) || overlap(rl, rk) ||
        overlap(rl, rv) || overlap(ro, rl))
        return ATTN_E_ALIAS;
    if (bm && (overlap(ro, range_of(bm, mb)) || overlap(rl, range_of(bm, mb)))) return ATTN_E_ALIAS;
    attn::FwdParams p{q, k, v, o, lse, dense_layout(B, H, N, causal, bm, mask_heads), N, d, dtype, scale, stream};
    return attn::launch_fwd(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

// from_scratch: the D buffer is the library's fixed device scratch
// (attn_bwd_noalloc); workspace and workspace_bytes are then ignored.
int bwd_dense(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, int B, int H, int N, int d, const uint8_t* bm, int mask_heads,
              int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, bool from_scratch,
              void* stream) {
    int64_t rows = 0, elems = 0;
    int st = check_common(B, H, N, d, causal, scale, dtype, &rows, &elems);
    if (st != ATTN_OK) return st;
    if (rows == 0) return ATTN_OK;
    size_t mb = 0;
    if (bm) {
        mb = mask_bytes(B, H, N, mask_heads);
        if (mb == 0) return ATTN_E_SHAPE;
    }
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
    if (from_scratch) workspace = nullptr;
    else if (!workspace) return ATTN_E_WORKSPACE;
    const void* a16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : a16)
        if (!aligned(p, 16)) return ATTN_E_ALIGN;
    if (!aligned(lse, 4)) return ATTN_E_ALIGN;
    const size_t ws_need = attn::bwd_workspace_bytes_rows(rows);
    if (from_scratch) {
        if (ws_need > attn::kScratchBytes) return ATTN_E_TOO_LARGE;
    } else if (workspace_bytes < ws_need) {
        return ATTN_E_WORKSPACE;
    }
    const size_t tb = (size_t)elems * 2, lb = (size_t)rows * 4;
    const Range ins[] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), range_of(o, tb),
                         range_of(dout, tb), range_of(lse, lb), range_of(bm, mb)};
    const Range outs[] = {range_of(dq, tb), range_of(dk, tb), range_of(dv, tb),
                          range_of(workspace, from_scratch ? 0 : ws_need)};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return i == 3 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return j == 3 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
    }
    // Every row's D is written by the dQ kernel before the dK/dV kernel reads
    // it, so the scratch needs no clearing between calls.
    if (from_scratch && attn::scratch_for_stream(stream, &workspace) != hipSuccess) return ATTN_E_HIP;
    attn::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace,
                      dense_layout(B, H, N, causal, bm, mask_heads), N, N, d, dtype, scale, stream};
    return attn::launch_bwd(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
             int d, int causal, float scale, int dtype, void* stream) {
    return fwd_dense(q, k, v, o, lse, B, H, N, d, nullptr, 0, causal, scale, dtype, stream);
}

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                         int d, const uint8_t* block_mask, int mask_heads, int causal, float scale, int dtype,
                         void* stream) {
    if ((int64_t)B * H * N > 0 && !block_mask) return ATTN_E_NULL;
    return fwd_dense(q, k, v, o, lse, B, H, N, d, block_mask, mask_heads, causal, scale, dtype, stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
    if (B < 0 || H < 0 || N < 0 || d < 0) return (size_t)-1;
    if ((int64_t)B * H * N == 0) return 0;
    (void)d;
    return attn::bwd_workspace_bytes_rows((int64_t)B * H * N);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, nullptr, 0, causal, scale, dtype, workspace,
                     workspace_bytes, false, stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                     float scale, int dtype, void* stream) {
    return bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, nullptr, 0, causal, scale, dtype, nullptr, 0,
                     true, stream);
}

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                         const uint8_t* block_mask, int mask_heads, int causal, float scale, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if ((int64_t)B * H * N > 0 && !block_mask) return ATTN_E_NULL;
    return bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, block_mask, mask_heads, causal, scale, dtype,
                     workspace, workspace_bytes, false, stream);
}

namespace {

// Checks shared by the packed variable-length entry points.
int check_varlen(const int* cu_q, const int* cu_k, int batch, int H, int total_q, int total_k,
                 int max_q, int max_k, int d, int causal, int wl, int wr, float scale, int dtype) {
    if (batch < 0 || H < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0) return ATTN_E_SHAPE;
    if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_E_UNSUPPORTED;
    if (wl < -1 || wr < -1) return ATTN_E_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_E_UNSUPPORTED;
    if (batch == INT32_MAX) return ATTN_E_SHAPE;  // batch + 1 offsets must be addressable
    if ((int64_t)total_q + total_k > ((int64_t)1 << 30)) return ATTN_E_SHAPE;
    if (batch > 0 && (!cu_q || !cu_k)) return ATTN_E_NULL;
    if (!aligned(cu_q, 4) || !aligned(cu_k, 4)) return ATTN_E_ALIGN;
    return ATTN_OK;
}

// A window reaching total_q + total_k positions or more covers every key of
// every row (|pos - j| < total_q + total_k), so it is the unbounded window -1.
// check_varlen bounds total_q + total_k by 2^30, which keeps the device's
// position and window arithmetic (pos +- window) inside int32.
int clamp_window(int w, int total_q, int total_k) {
    return (int64_t)w >= (int64_t)total_q + total_k ? -1 : w;
}

attn::SeqLayout varlen_layout(const int* cu_q, const int* cu_k, int batch, int H, int total_q, int total_k,
                              int causal, int wl, int wr) {
    wl = clamp_window(wl, total_q, total_k);
    wr = causal ? 0 : clamp_window(wr, total_q, total_k);
    return attn::SeqLayout{1, batch, H, 0, cu_q, cu_k, total_q, total_k, wl, wr, nullptr, 0, 0};
}

}  // namespace

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int batch, int H, int total_q, int total_k, int max_seqlen_q,
                    int d, int causal, int window_left, int window_right, float scale, int dtype, void* stream) {
    int st = check_varlen(cu_seqlens_q, cu_seqlens_k, batch, H, total_q, total_k, max_seqlen_q, 0, d, causal,
                          window_left, window_right, scale, dtype);
    if (st != ATTN_OK) return st;
    if ((int64_t)batch * H == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_OK;
    if (!q || !o || !lse || (total_k > 0 && (!k || !v))) return ATTN_E_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return ATTN_E_ALIGN;
    const size_t qb = (size_t)H * total_q * d * 2, kb = (size_t)H * total_k * d * 2, lb = (size_t)H * total_q * 4;
    const Range rq = range_of(q, qb), rk = range_of(k, kb), rv = range_of(v, kb);
    const Range ro = range_of(o, qb), rl = range_of(lse, lb);
    const Range rcq = range_of(cu_seqlens_q, (size_t)(batch + 1) * 4), rck = range_of(cu_seqlens_k, (size_t)(batch + 1) * 4);
    for (const Range& out : {ro, rl})
        for (const Range& in : {rq, rk, rv, rcq, rck})
            if (overlap(out, in)) return ATTN_E_ALIAS;
    if (overlap(ro, rl)) return ATTN_E_ALIAS;
    attn::FwdParams p{q, k, v, o, lse,
                      varlen_layout(cu_seqlens_q, cu_seqlens_k, batch, H, total_q, total_k, causal, window_left,
                                    window_right),
                      max_seqlen_q, d, dtype, scale, stream};
    return attn::launch_fwd(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_fwd_unfused_workspace_bytes(int B, int H, int N) {
    if (B < 0 || H < 0 || N < 0) return (size_t)-1;
    if ((int64_t)B * H * N == 0) return 0;
    if ((int64_t)N > (int64_t)1 << 24 || (int64_t)B * H > 65535) return (size_t)-1;
    return attn::unfused_workspace_bytes(B, H, N);
}

int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                     int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    int64_t rows = 0, elems = 0;
    int st = check_common(B, H, N, d, causal, scale, dtype, &rows, &elems);
    if (st != ATTN_OK) return st;
    if (rows == 0) return ATTN_OK;
    if ((int64_t)B * H > 65535 || (int64_t)N > (int64_t)1 << 24 || rows > INT32_MAX) return ATTN_E_SHAPE;
    if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
    if (!workspace) return ATTN_E_WORKSPACE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(workspace, 16))
        return ATTN_E_ALIGN;
    const size_t need = attn::unfused_workspace_bytes(B, H, N);
    if (workspace_bytes < need) return ATTN_E_WORKSPACE;
    const size_t tb = (size_t)elems * 2, lb = (size_t)rows * 4;
    const Range ins[] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
    const Range outs[] = {range_of(o, tb), range_of(lse, lb), range_of(workspace, need)};
    for (int i = 0; i < 3; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return i == 2 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return j == 2 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
    }
    attn::UnfusedParams p{q, k, v, o, lse, workspace, B, H, N, d, causal, dtype, scale, stream};
    return attn::launch_unfused(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_bwd_varlen_workspace_bytes(int H, int total_q) {
    if (H < 0 || total_q < 0) return (size_t)-1;
    if ((int64_t)H * total_q == 0) return 0;
    return attn::bwd_workspace_bytes_rows((int64_t)H * total_q);
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, const int* cu_seqlens_q, const int* cu_seqlens_k, int batch,
                    int H, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                    int window_left, int window_right, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int st = check_varlen(cu_seqlens_q, cu_seqlens_k, batch, H, total_q, total_k, max_seqlen_q, max_seqlen_k, d,
                          causal, window_left, window_right, scale, dtype);
    if (st != ATTN_OK) return st;
    if ((int64_t)batch * H == 0 || (total_q == 0 && total_k == 0)) return ATTN_OK;
    const bool has_q = total_q > 0, has_k = total_k > 0;
    if ((has_q && (!q || !o || !dout || !lse || !dq)) || (has_k && (!k || !v || !dk || !dv))) return ATTN_E_NULL;
    const size_t ws_need = attn::bwd_workspace_bytes_rows((int64_t)H * total_q);
    if (ws_need > 0 && !workspace) return ATTN_E_WORKSPACE;
    const void* a16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* ptr : a16)
        if (!aligned(ptr, 16)) return ATTN_E_ALIGN;
    if (!aligned(lse, 4)) return ATTN_E_ALIGN;
    if (workspace_bytes < ws_need) return ATTN_E_WORKSPACE;
    const size_t qb = (size_t)H * total_q * d * 2, kb = (size_t)H * total_k * d * 2, lb = (size_t)H * total_q * 4;
    const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb), range_of(o, qb), range_of(dout, qb),
                         range_of(lse, lb), range_of(cu_seqlens_q, (size_t)(batch + 1) * 4),
                         range_of(cu_seqlens_k, (size_t)(batch + 1) * 4)};
    const Range outs[] = {range_of(dq, qb), range_of(dk, kb), range_of(dv, kb), range_of(workspace, ws_need)};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return i == 3 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return j == 3 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
    }
    attn::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace,
                      varlen_layout(cu_seqlens_q, cu_seqlens_k, batch, H, total_q, total_k, causal, window_left,
                                    window_right),
                      max_seqlen_q, max_seqlen_k, d, dtype, scale, stream};
    return attn::launch_bwd(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // extern "C"
