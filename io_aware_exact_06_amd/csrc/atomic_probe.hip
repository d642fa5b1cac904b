// atomic_probe.hip -- throughput of fp32 atomic adds into a dQ accumulator in
// the pattern a key-stationary backward would use, against plain stores of the
// same bytes.
//
// Grid: heads x 128-key groups, renumbered as the attention kernels do
// (xcd_contiguous: each XCD receives one contiguous range, i.e. the groups of
// few heads at a time).  Group (head, kt) adds one 64 x d fp32 tile (32 KB at
// d = 128) into dq[head] for every 64-row query tile it would visit: query
// tiles 2 kt .. N/64 - 1 when causal, all of them otherwise.  Every wave
// instruction covers 64 consecutive floats (global_atomic_add_f32 with no
// return value).
//
// Usage: atomic_probe     prints one JSON object on stdout (shape of the
//                         benchmark workload: 32 heads, N = 8192, d = 128).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

__device__ inline int xcd_contiguous(int b, int n) {
    const int q = n >> 3, r = n & 7;
    const int xcd = b & 7, local = b >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

constexpr int kRows = 64;

template <bool ATOMIC>
__global__ __launch_bounds__(256) void add_tiles(float* dq, int nkt, int nqt, int causal, int d) {
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const int head = item / nkt, kt = item % nkt;
    float* base = dq + (size_t)head * nqt * kRows * d;
    const float v = 1.0f / (1 + threadIdx.x);
    for (int qt = causal ? 2 * kt : 0; qt < nqt; ++qt) {
        float* t = base + (size_t)qt * kRows * d;
#pragma unroll 4
        for (int i = threadIdx.x; i < kRows * d; i += 256) {
            if (ATOMIC) unsafeAtomicAdd(t + i, v);
            else t[i] = v;
        }
    }
}

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "atomic_probe: %s failed: %s\n", #x, hipGetErrorString(e_));  \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

}  // namespace

int main() {
    const int H = 32, N = 8192, d = 128;
    const int nkt = N / 128, nqt = N / kRows;
    float* dq = nullptr;
    CHECK(hipMalloc(&dq, (size_t)H * N * d * sizeof(float)));
    CHECK(hipMemset(dq, 0, (size_t)H * N * d * sizeof(float)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    printf("{\"heads\": %d, \"N\": %d, \"d\": %d", H, N, d);
    for (int causal = 1; causal >= 0; --causal) {
        double tiles = 0;
        for (int kt = 0; kt < nkt; ++kt) tiles += nqt - (causal ? 2 * kt : 0);
        const double bytes = tiles * H * kRows * d * sizeof(float);
        for (int atomic = 1; atomic >= 0; --atomic) {
            float best = 1e30f;
            for (int rep = 0; rep < 4; ++rep) {
                CHECK(hipEventRecord(e0, 0));
                if (atomic)
                    hipLaunchKernelGGL(add_tiles<true>, dim3(H * nkt), dim3(256), 0, 0, dq, nkt, nqt, causal, d);
                else
                    hipLaunchKernelGGL(add_tiles<false>, dim3(H * nkt), dim3(256), 0, 0, dq, nkt, nqt, causal, d);
                CHECK(hipGetLastError());
                CHECK(hipEventRecord(e1, 0));
                CHECK(hipEventSynchronize(e1));
                float ms = 0.f;
                CHECK(hipEventElapsedTime(&ms, e0, e1));
                if (ms < best) best = ms;
            }
            printf(", \"%s_%s\": {\"ms\": %.4f, \"gb\": %.3f, \"tb_per_s\": %.3f}", causal ? "causal" : "full",
                   atomic ? "atomic_add_f32" : "store", best, bytes / 1e9, bytes / best / 1e9);
        }
    }
    printf("}\n");
    CHECK(hipFree(dq));
    return 0;
}
