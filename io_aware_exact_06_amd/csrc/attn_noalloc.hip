// attn_noalloc.hip -- the fixed device scratch behind attn_bwd_noalloc.
//
// attn_bwd needs a caller-supplied workspace for the per-row terms
// -D_i (D_i = <dO_i, O_i>), which the dQ kernel writes and the dK/dV kernel reads.
// Callers that cannot allocate device memory (code under graph capture,
// tight serving loops) use attn_bwd_noalloc instead.  Its D buffer is the
// file-scope array below: every GPU the library runs on holds one copy of it,
// at its own address, until the process ends.
//
// Host code never passes the array's name to a kernel: in host code that name
// is a stand-in, not a device address.  scratch_for_stream() looks the
// address up once per device with hipGetSymbolAddress (with that device
// current) and the callers pass only that pointer on.

#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_launch.h"

static __device__ __align__(256) float scratch[attn::kScratchBytes / sizeof(float)];

namespace attn {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // address of `scratch` on each device; nullptr until looked up

}  // namespace

hipError_t scratch_for_stream(void* stream, void** ptr) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice((hipStream_t)stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace attn
