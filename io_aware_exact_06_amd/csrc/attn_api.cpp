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
    if (!isfinite(scale) || scale < 0.f) return ATTN_E_UNSUPPORTED;
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
        default: return "unknown status";
    }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
             int d, int causal, float scale, int dtype, void* stream) {
    int64_t rows = 0, elems = 0;
    int st = check_common(B, H, N, d, causal, scale, dtype, &rows, &elems);
    if (st != ATTN_OK) return st;
    if (rows == 0) return ATTN_OK;
    if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return ATTN_E_ALIGN;
    const size_t tb = (size_t)elems * 2, lb = (size_t)rows * 4;
    const Range rq = range_of(q, tb), rk = range_of(k, tb), rv = range_of(v, tb);
    const Range ro = range_of(o, tb), rl = range_of(lse, lb);
    if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) || overlap(rl, rk) ||
        overlap(rl, rv) || overlap(ro, rl))
        return ATTN_E_ALIAS;
    attn::FwdParams p{q, k, v, o, lse, B, H, N, d, causal, dtype, scale, stream};
    return attn::launch_fwd(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
    if (B < 0 || H < 0 || N < 0 || d < 0) return (size_t)-1;
    if ((int64_t)B * H * N == 0) return 0;
    (void)d;
    return attn::bwd_workspace_bytes(B, H, N);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    int64_t rows = 0, elems = 0;
    int st = check_common(B, H, N, d, causal, scale, dtype, &rows, &elems);
    if (st != ATTN_OK) return st;
    if (rows == 0) return ATTN_OK;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
    if (!workspace) return ATTN_E_WORKSPACE;
    const void* a16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : a16)
        if (!aligned(p, 16)) return ATTN_E_ALIGN;
    if (!aligned(lse, 4)) return ATTN_E_ALIGN;
    const size_t ws_need = attn::bwd_workspace_bytes(B, H, N);
    if (workspace_bytes < ws_need) return ATTN_E_WORKSPACE;
    const size_t tb = (size_t)elems * 2, lb = (size_t)rows * 4;
    const Range ins[] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), range_of(o, tb),
                         range_of(dout, tb), range_of(lse, lb)};
    const Range outs[] = {range_of(dq, tb), range_of(dk, tb), range_of(dv, tb),
                          range_of(workspace, ws_need)};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return i == 3 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return j == 3 ? ATTN_E_WORKSPACE : ATTN_E_ALIAS;
    }
    attn::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace,
                      B, H, N, d, causal, dtype, scale, stream};
    return attn::launch_bwd(p) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // extern "C"
