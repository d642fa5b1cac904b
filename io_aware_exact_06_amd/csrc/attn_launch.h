// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and
// the kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kDtypeF16 = 0;
constexpr int kDtypeBF16 = 1;

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N, d, causal, dtype;
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
    float* dq_acc;  // fp32 [B, H, N, d], part of the caller's workspace
    float* delta;   // fp32 [B, H, N], part of the caller's workspace
    int B, H, N, d, causal, dtype;
    float scale;
    void* stream;
};

// Byte offsets of the backward workspace regions (256-byte aligned).
struct BwdWorkspaceLayout {
    size_t dq_acc_offset, delta_offset, total;
};

inline size_t round_up_256(size_t x) { return (x + 255) & ~(size_t)255; }

inline BwdWorkspaceLayout bwd_workspace_layout(int64_t B, int64_t H, int64_t N, int64_t d) {
    BwdWorkspaceLayout w;
    const size_t rows = (size_t)(B * H * N);
    w.dq_acc_offset = 0;
    w.delta_offset = round_up_256(rows * (size_t)d * sizeof(float));
    w.total = w.delta_offset + round_up_256(rows * sizeof(float));
    return w;
}

hipError_t launch_fwd(const FwdParams& p);
hipError_t launch_bwd(const BwdParams& p);

}  // namespace attn
