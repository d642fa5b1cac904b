// attn_unfused.hip -- the standard, unfused attention forward, kept as a
// measurable baseline for the fused kernels' IO claim.
//
// It performs the three passes the hotdry blog's section "传统注意力计算的内存
// 带宽瓶颈" lists, each as its own kernel with its intermediate in device
// memory:
//   1. S = scale * Q K^T, written to HBM as fp32 [BH, N, N];
//   2. P = softmax(S) row by row (the row maximum is subtracted first, as in
//      the stable_softmax example of the snabindia page, section 2.2; causal
//      entries j > i get P = 0), written as 16-bit [BH, N, N], with lse;
//   3. O = P V.
// Every score is therefore written once and read twice, and every
// probability written once and read once -- the O(N^2) traffic that the
// fused forward never generates.  S is computed in full even when causal (the
// standard flow does not skip the upper triangle).

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;  // rows and columns of a score tile / rows of an output tile
constexpr int kBK = 64;     // keys per step of the P V product

// ---- pass 1: S = scale * Q K^T (fp32), one 128 x 128 tile per work group -------------
template <class T, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void unfused_scores_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, float* __restrict__ S,
                           int N, int ntile, float scale) {
    constexpr int STR = LdsStride<D>::value, KS = D / 16;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * STR];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n32 = lane & 31, h = lane >> 5;
    const int bh = blockIdx.y;
    const int qt = blockIdx.x / ntile, kt = blockIdx.x % ntile;
    const uint16_t* Qh = Q + (int64_t)bh * N * D;
    const uint16_t* Kh = K + (int64_t)bh * N * D;
    float* Sh = S + (int64_t)bh * N * N;
    const int q0 = qt * kTile, k0 = kt * kTile;
    // K tile rows (clamped: rows past N repeat row N-1 and their scores are not stored)
    for (int c = tid; c < kTile * (D / 8); c += kThreads) {
        const int r = c / (D / 8), col = c % (D / 8);
        *(u32x4*)(Ks + r * STR + 8 * col) = *(const u32x4*)(Kh + (int64_t)min(k0 + r, N - 1) * D + 8 * col);
    }
    const int qrow = q0 + 32 * w + n32;
    u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4*)(Qh + (int64_t)min(qrow, N - 1) * D + 16 * ks + 8 * h);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
        const uint16_t* kp = Ks + (kb * 32 + n32) * STR + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32<T>(*(const u32x4*)(kp + 16 * ks), qf[ks], s);
        // lane holds query qrow, keys k0 + 32 kb + 8 (e/4) + 4 h + (0..3): four consecutive keys per group
        if (qrow < N) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int key = k0 + kb * 32 + 8 * g + 4 * h;
                const f32x4 v4 = {s[4 * g] * scale, s[4 * g + 1] * scale, s[4 * g + 2] * scale, s[4 * g + 3] * scale};
                if ((N & 3) == 0 && key + 3 < N) {  // 16-byte aligned when N % 4 == 0
                    *(f32x4*)(Sh + (int64_t)qrow * N + key) = v4;
                } else {
                    for (int i = 0; i < 4; ++i)
                        if (key + i < N) Sh[(int64_t)qrow * N + key + i] = v4[i];
                }
            }
        }
    }
}

// ---- pass 2: P = softmax(S) per row, lse; one wave per row --------------------------------
template <class T>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void unfused_softmax_kernel(const float* __restrict__ S, uint16_t* __restrict__ P, float* __restrict__ LSE, int N,
                            int rows, int causal) {
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int i = row % N;                         // row index inside its head
    const int nvis = causal ? i + 1 : N;           // visible keys: 0 .. nvis-1
    const float* s = S + (int64_t)row * N;
    uint16_t* p = P + (int64_t)row * N;
    float m = kNegInf;
    for (int j = lane; j < nvis; j += 64) m = fmaxf(m, s[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.f;
    for (int j = lane; j < nvis; j += 64) l += __builtin_amdgcn_exp2f((s[j] - m) * kLog2e);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    const float inv = 1.f / l;
    for (int j = 2 * lane; j < N; j += 128) {
        const float p0 = j < nvis ? __builtin_amdgcn_exp2f((s[j] - m) * kLog2e) * inv : 0.f;
        const float p1 = j + 1 < nvis ? __builtin_amdgcn_exp2f((s[j + 1] - m) * kLog2e) * inv : 0.f;
        const uint32_t pk = pack2<T>(p0, p1);
        if ((N & 1) == 0) {  // 4-byte aligned pairs when N is even
            *(uint32_t*)(p + j) = pk;
        } else {
            p[j] = (uint16_t)(pk & 0xffffu);
            if (j + 1 < N) p[j + 1] = (uint16_t)(pk >> 16);
        }
    }
    if (lane == 0) LSE[row] = m + logf(l);
}

// ---- pass 3: O = P V, 128 rows per work group, keys in steps of 64 ------------------------
template <class T, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void unfused_pv_kernel(const uint16_t* __restrict__ P, const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                       int N, int ntq) {
    constexpr int STR = LdsStride<D>::value, DB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kBK * STR];
    __shared__ __attribute__((aligned(16))) uint16_t Os[kTile * STR];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n32 = lane & 31, h = lane >> 5;
    const int bh = blockIdx.x / ntq, q0 = (blockIdx.x % ntq) * kTile;
    const uint16_t* Ph = P + (int64_t)bh * N * N;
    const uint16_t* Vh = V + (int64_t)bh * N * D;
    const int qrow = q0 + 32 * w + n32;
    const int prow = min(qrow, N - 1);
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    const int tr_off = tr_lane_offset<STR>(lane);
    for (int k0 = 0; k0 < N; k0 += kBK) {
        __syncthreads();
        for (int c = tid; c < kBK * (D / 8); c += kThreads) {
            const int r = c / (D / 8), col = c % (D / 8);
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4*)(Vs + r * STR + 8 * col) = k0 + r < N ? *(const u32x4*)(Vh + (int64_t)(k0 + r) * D + 8 * col) : z;
        }
        __syncthreads();
        // B operand P^T: lane (query, h) takes keys k0 + 16 t' + 8 h .. +7 of its row; the
        // matching rows of V^T come from the transpose read (row order 8(e/4) + 4h + e%4 per
        // 16-key step), so the P values are gathered in that order.
#pragma unroll
        for (int st = 0; st < kBK / 16; ++st) {
            u32x4 b;
            const int kb0 = k0 + 16 * st;
            const uint16_t* pr = Ph + (int64_t)prow * N;
            if ((N & 3) == 0 && kb0 + 16 <= N) {  // two aligned 8-byte runs of 4 keys
                const u32x2 lo = *(const u32x2*)(pr + kb0 + 4 * h);
                const u32x2 hi = *(const u32x2*)(pr + kb0 + 8 + 4 * h);
                b[0] = lo[0], b[1] = lo[1], b[2] = hi[0], b[3] = hi[1];
            } else {
                uint16_t pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = kb0 + 8 * (e >> 2) + 4 * h + (e & 3);
                    pv[e] = key < N ? pr[key] : (uint16_t)0;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) b[i] = (uint32_t)pv[2 * i] | ((uint32_t)pv[2 * i + 1] << 16);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = mfma32<T>(tr_operand<STR>(Vs + tr_off, 16 * st, 32 * db), b, oacc[db]);
        }
    }
    // O rows are already normalised (P is); stage and store row-contiguously
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 pk = {pack2<T>(oacc[db][4 * g], oacc[db][4 * g + 1]), pack2<T>(oacc[db][4 * g + 2], oacc[db][4 * g + 3])};
            *(u32x2*)(Os + (32 * w + n32) * STR + 32 * db + 8 * g + 4 * h) = pk;
        }
    __syncthreads();
    uint16_t* Oh = O + (int64_t)bh * N * D;
    for (int c = tid; c < kTile * (D / 8); c += kThreads) {
        const int r = c / (D / 8), col = c % (D / 8);
        if (q0 + r < N) *(u32x4*)(Oh + (int64_t)(q0 + r) * D + 8 * col) = *(const u32x4*)(Os + r * STR + 8 * col);
    }
}

template <class T, int D>
hipError_t launch_unfused_t(const UnfusedParams& p) {
    const int64_t bh = (int64_t)p.B * p.H;
    const int nt = (p.N + kTile - 1) / kTile;
    if (bh > 65535 || (int64_t)nt * nt > 0x7fffffff || bh * p.N > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipStream_t st = (hipStream_t)p.stream;
    float* S = (float*)p.workspace;
    uint16_t* P = (uint16_t*)((char*)p.workspace + unfused_score_bytes(p.B, p.H, p.N));
    hipLaunchKernelGGL((unfused_scores_kernel<T, D>), dim3((unsigned)(nt * nt), (unsigned)bh), dim3(kThreads), 0, st,
                       (const uint16_t*)p.q, (const uint16_t*)p.k, S, p.N, nt, p.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rows = (int)(bh * p.N);
    hipLaunchKernelGGL((unfused_softmax_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, st, S, P,
                       p.lse, p.N, rows, p.causal);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((unfused_pv_kernel<T, D>), dim3((unsigned)(bh * nt)), dim3(kThreads), 0, st, P,
                       (const uint16_t*)p.v, (uint16_t*)p.o, p.N, nt);
    return hipGetLastError();
}

template <class T>
hipError_t launch_unfused_d(const UnfusedParams& p) {
    return p.d == 64 ? launch_unfused_t<T, 64>(p) : launch_unfused_t<T, 128>(p);
}

}  // namespace

hipError_t launch_unfused(const UnfusedParams& p) {
    return p.dtype == kDtypeBF16 ? launch_unfused_d<BF16>(p) : launch_unfused_d<F16>(p);
}

}  // namespace attn
