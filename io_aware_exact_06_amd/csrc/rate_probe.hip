// rate_probe.hip -- throughput of the three instruction kinds the attention
// kernels are made of, measured on the GPU they run on: the transcendental
// v_exp_f32 (one per score element), the fp32 FMA (unpacked: this library is
// built without packed fp32), and the 32x32x16 bf16 MFMA.
//
// Every work group times itself with two counters: s_memtime (shader clock
// cycles) and s_memrealtime (a fixed 100 MHz clock).  The grid is two work
// groups of four waves per CU, all resident at once, so a group's cycle count
// is the kernel's; rates come out per CU per shader cycle, independent of
// the clock, and the ratio of the two counters is the clock the part ran at.
//
// Usage: rate_probe            prints one JSON object on stdout.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kGroupsPerCu = 2;
constexpr int kChains = 16;  // independent chains per lane: enough to cover the latency of both ops

// One record per work group: shader cycles, 100 MHz ticks.  Lane 0 of wave 0
// writes it with vector stores (a per-lane address).
__device__ inline void record(uint64_t* out, uint64_t c0, uint64_t r0) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c1 - c0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

__global__ __launch_bounds__(kWaves * 64) void exp_kernel(uint64_t* out, float* sink, int iters) {
    float x[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) x[i] = 0.001f * (threadIdx.x + i);
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < kChains; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);  // stays in (0, 1]
    __syncthreads();
    record(out, c0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += x[i];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(kWaves * 64) void fma_kernel(uint64_t* out, float* sink, int iters, float a, float b) {
    float x[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) x[i] = 0.001f * (threadIdx.x + i);
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < kChains; ++i) x[i] = __builtin_fmaf(x[i], a, b);
    __syncthreads();
    record(out, c0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += x[i];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(kWaves * 64) void mfma_kernel(uint64_t* out, float* sink, int iters) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (threadIdx.x + i));
        b[i] = (__bf16)(0.002f * (threadIdx.x - i));
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    __syncthreads();
    record(out, c0, r0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

struct Result {
    double per_clk_per_cu;  // operations (or flops) per shader cycle per CU
    double mhz;             // shader clock during the run
};

// ops_per_group: operations one work group performs.
Result summarize(const uint64_t* rec, int groups, double ops_per_group) {
    uint64_t cyc = 0, rt = 0;
    for (int g = 0; g < groups; ++g) {
        if (rec[2 * g] > cyc) cyc = rec[2 * g];
        if (rec[2 * g + 1] > rt) rt = rec[2 * g + 1];
    }
    Result r;
    r.per_clk_per_cu = ops_per_group * kGroupsPerCu / (double)cyc;
    r.mhz = rt ? (double)cyc / ((double)rt / 100.0) : 0.0;  // rt counts 100 MHz ticks
    return r;
}

#define CHECK(x)                                                                            \
    do {                                                                                    \
        hipError_t e_ = (x);                                                                \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "rate_probe: %s failed: %s\n", #x, hipGetErrorString(e_));      \
            return 1;                                                                       \
        }                                                                                   \
    } while (0)

}  // namespace

int main() {
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    const int groups = cus * kGroupsPerCu;
    const int threads = kWaves * 64;
    uint64_t* rec_d = nullptr;
    float* sink = nullptr;
    CHECK(hipMalloc(&rec_d, sizeof(uint64_t) * 2 * groups));
    CHECK(hipMalloc(&sink, sizeof(float) * groups * threads));
    uint64_t* rec = new uint64_t[2 * groups];

    const int it_exp = 20000, it_fma = 40000, it_mfma = 4000;
    Result r_exp, r_fma, r_mfma;
    for (int rep = 0; rep < 2; ++rep) {  // the first pass warms the clock up
        hipLaunchKernelGGL(exp_kernel, dim3(groups), dim3(threads), 0, 0, rec_d, sink, it_exp);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        CHECK(hipMemcpy(rec, rec_d, sizeof(uint64_t) * 2 * groups, hipMemcpyDeviceToHost));
        r_exp = summarize(rec, groups, (double)it_exp * kChains * threads);

        hipLaunchKernelGGL(fma_kernel, dim3(groups), dim3(threads), 0, 0, rec_d, sink, it_fma, 0.999f, 0.001f);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        CHECK(hipMemcpy(rec, rec_d, sizeof(uint64_t) * 2 * groups, hipMemcpyDeviceToHost));
        r_fma = summarize(rec, groups, (double)it_fma * kChains * threads);

        hipLaunchKernelGGL(mfma_kernel, dim3(groups), dim3(threads), 0, 0, rec_d, sink, it_mfma);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        CHECK(hipMemcpy(rec, rec_d, sizeof(uint64_t) * 2 * groups, hipMemcpyDeviceToHost));
        r_mfma = summarize(rec, groups, (double)it_mfma * 4 * kWaves * 32.0 * 32.0 * 16.0 * 2.0);
    }
    printf("{\"cus\": %d, \"exp_per_clk_per_cu\": %.3f, \"exp_mhz\": %.0f, "
           "\"fma_f32_per_clk_per_cu\": %.3f, \"fma_mhz\": %.0f, "
           "\"mfma_bf16_flop_per_clk_per_cu\": %.1f, \"mfma_mhz\": %.0f}\n",
           cus, r_exp.per_clk_per_cu, r_exp.mhz, r_fma.per_clk_per_cu, r_fma.mhz, r_mfma.per_clk_per_cu, r_mfma.mhz);
    delete[] rec;
    CHECK(hipFree(rec_d));
    CHECK(hipFree(sink));
    return 0;
}
