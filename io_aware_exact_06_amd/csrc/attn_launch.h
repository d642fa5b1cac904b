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
    float* delta;  // fp32 [B, H, N] row terms D_i = <dO_i, O_i>: the caller's workspace
    int B, H, N, d, causal, dtype;
    float scale;
    void* stream;
};

// Bytes of backward workspace: one fp32 D per query row, rounded up to 256.
inline size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
    return (((size_t)(B * H * N) * sizeof(float)) + 255) & ~(size_t)255;
}

hipError_t launch_fwd(const FwdParams& p);
hipError_t launch_bwd(const BwdParams& p);

}  // namespace attn
