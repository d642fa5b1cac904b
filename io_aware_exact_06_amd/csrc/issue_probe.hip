// issue_probe.hip -- how much vector work hides under the 32x32x16 bf16 MFMA.
//
// Every kernel runs a loop of 4 independent MFMA accumulators, each MFMA
// followed by R independent fp32 FMAs (16 chains) or R v_exp_f32, or the
// vector work alone.  One work group of four waves per CU gives one wave per
// SIMD, two groups give two; all groups are resident at once and time
// themselves with s_memtime (shader cycles).  The figure printed is shader
// cycles per (MFMA + R operations) per wave slot, i.e. per MFMA of one SIMD.
//
// Usage: issue_probe     prints one JSON object on stdout.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kIters = 2000;

// MODE 0: MFMA + R FMA; 1: MFMA + R exp; 2: R FMA only; 3: R exp only.
template <int MODE, int R>
__global__ __launch_bounds__(256) void probe(uint64_t* out, float* sink, int iters, float a, float b) {
    bf16x8 x, y;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[i] = (__bf16)(0.001f * (threadIdx.x + i));
        y[i] = (__bf16)(0.002f * i);
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.001f * (threadIdx.x + i);
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (MODE <= 1) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[j], 0, 0, 0);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = (j * R + r) & 15;
                if (MODE == 0 || MODE == 2) v[i] = __builtin_fmaf(v[i], a, b);
                else v[i] = __builtin_amdgcn_exp2f(-v[i]);  // stays in (0, 1]
            }
        }
    }
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) out[blockIdx.x] = c1 - c0;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
#pragma unroll
    for (int i = 0; i < 16; ++i) s += v[i];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "issue_probe: %s failed: %s\n", #x, hipGetErrorString(e_));  \
            return -1.0;                                                                 \
        }                                                                                \
    } while (0)

// Cycles per (MFMA + R ops) per wave slot with `gpc` groups per CU.
template <int MODE, int R>
double run(int cus, int gpc, uint64_t* out_d, float* sink, uint64_t* out) {
    const int groups = cus * gpc;
    for (int rep = 0; rep < 2; ++rep) {  // the first pass warms the clock up
        hipLaunchKernelGGL((probe<MODE, R>), dim3(groups), dim3(256), 0, 0, out_d, sink, kIters, 0.999f, 0.001f);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
    }
    CHECK(hipMemcpy(out, out_d, sizeof(uint64_t) * groups, hipMemcpyDeviceToHost));
    uint64_t mx = 0;
    for (int g = 0; g < groups; ++g) mx = out[g] > mx ? out[g] : mx;
    return (double)mx / (kIters * 4.0 * gpc);
}

}  // namespace

int main() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
    const int cus = prop.multiProcessorCount;
    uint64_t* out_d = nullptr;
    float* sink = nullptr;
    if (hipMalloc(&out_d, sizeof(uint64_t) * cus * 2) != hipSuccess) return 1;
    if (hipMalloc(&sink, sizeof(float) * cus * 2 * 256) != hipSuccess) return 1;
    uint64_t* out = new uint64_t[cus * 2];
    printf("{\"unit\": \"shader cycles per MFMA (or per R ops alone) per SIMD\"");
    for (int gpc = 1; gpc <= 2; ++gpc) {
        const double r[] = {
            run<0, 0>(cus, gpc, out_d, sink, out),  run<0, 4>(cus, gpc, out_d, sink, out),
            run<0, 6>(cus, gpc, out_d, sink, out),  run<0, 8>(cus, gpc, out_d, sink, out),
            run<0, 12>(cus, gpc, out_d, sink, out), run<1, 2>(cus, gpc, out_d, sink, out),
            run<1, 4>(cus, gpc, out_d, sink, out),  run<2, 16>(cus, gpc, out_d, sink, out),
            run<3, 8>(cus, gpc, out_d, sink, out)};
        for (double x : r)
            if (x < 0) return 1;
        printf(", \"waves_per_simd_%d\": {\"mfma\": %.1f, \"mfma_fma4\": %.1f, \"mfma_fma6\": %.1f, "
               "\"mfma_fma8\": %.1f, \"mfma_fma12\": %.1f, \"mfma_exp2\": %.1f, \"mfma_exp4\": %.1f, "
               "\"fma16_alone\": %.1f, \"exp8_alone\": %.1f}",
               gpc, r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7], r[8]);
    }
    printf("}\n");
    delete[] out;
    (void)hipFree(out_d);
    (void)hipFree(sink);
    return 0;
}
