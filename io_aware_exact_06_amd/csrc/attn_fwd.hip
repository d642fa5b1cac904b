// attn_fwd.hip -- fused exact-attention forward for gfx950.
//
// One work group owns BQ = 128 query rows of one (batch, head): four waves of
// 32 rows each.  The group streams the keys and values in tiles of BK = 64
// rows through LDS (double-buffered, next tile prefetched into registers
// while the current one is consumed), and each wave keeps, for its 32 rows,
// the running maximum m, the running sum l and the partial output in
// registers: the online softmax of the hotdry blog's section "3. 在线softmax
// 算法" (initialise m = -inf and l = 0; for every key block raise the maximum,
// rescale the running sum and the partial output when it grew, add the
// block's exponentials and their weighted values).  Only O and
// lse = scale * m + ln l leave the chip (section "1. 内核融合策略": write only
// the final output; section "4. 重计算" keeps one statistic per row).
//
// Orientation: every product is computed transposed, S^T = K Q^T and
// O^T = V^T P^T, on the 32x32x16 MFMA.  In that orientation the accumulator
// lane l always belongs to query row l % 32, so the row maximum, row sum and
// rescale factor are per-lane scalars; the only cross-lane step is one
// exchange between lane l and lane l ^ 32, which hold the two halves of the
// same row.  The exponentials come straight out of the S^T accumulator as
// the B operand of the P.V product (the key order inside an MFMA k-step is
// free, so the accumulator's own order is used), and V^T is read from the
// row-major V tile with the LDS transpose read.
//
// Causal masking (snabindia chapter 1: the causal call skips the upper
// triangle): key tiles beyond the group's last row are never loaded; a wave
// skips a loaded tile that lies wholly above its rows; only tiles that cross
// the diagonal or the end of the sequence are masked element by element.

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBQ = kWaves * kRowsPerWave;  // query rows per work group
constexpr int kBK = 64;                     // key rows per tile
constexpr int kThreads = kWaves * 64;

template <int D>
struct FwdShape {
    static constexpr int KS = D / 16;                 // MFMA k-steps of S^T over d
    static constexpr int DB = D / 32;                 // 32-row blocks of O^T
    static constexpr int KB = kBK / 32;               // 32-key blocks of a tile
    static constexpr int STR = LdsStride<D>::value;   // LDS row stride in elements
    static constexpr int CH = D / 8;                  // 16-byte chunks per row
    static constexpr int TILE = kBK * STR;            // elements per LDS tile
    static_assert(kBQ * STR <= 2 * TILE, "output staging must fit in the K buffers");
};

template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, int N, int ntq, float scale, float c) {
    using S = FwdShape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * S::TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * S::TILE];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n32 = lane & 31, h = lane >> 5;

    // Work item: (batch*head, query tile).  Each XCD gets a contiguous range;
    // within a head, causal tiles run longest first.
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bh = item / ntq;
    const int qt = CAUSAL ? ntq - 1 - item % ntq : item % ntq;
    const int64_t base = (int64_t)bh * N * D;
    const uint16_t* Qh = Q + base;
    const uint16_t* Kh = K + base;
    const uint16_t* Vh = V + base;
    const int q0 = qt * kBQ;
    const int wq0 = q0 + w * kRowsPerWave;  // first row of this wave
    const int qrow = wq0 + n32;             // the query row this lane accumulates

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop.
    u32x4 qf[S::KS];
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qf[ks] = qrow < N ? *(const u32x4*)(Qh + (int64_t)qrow * D + 16 * ks + 8 * h) : z;
    }

    const int kend = CAUSAL ? min(N, q0 + kBQ) : N;
    const int nkt = (kend + kBK - 1) / kBK;

    TileCopy<kBK, D, kThreads> kc, vc;
    kc.load(Kh, 0, N, tid);
    vc.load(Vh, 0, N, tid);
    kc.store(Ks, tid);
    vc.store(Vs, tid);
    __syncthreads();

    f32x16 oacc[S::DB];
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m = kNegInf;  // running maximum of the raw scores of row qrow
    float l = 0.f;      // this lane's share of the running sum (its 16 keys of every 32)

    const int tr_off = tr_lane_offset<S::STR>(lane);  // V^T read transposed from the V tile

    for (int jt = 0; jt < nkt; ++jt) {
        const int buf = (jt & 1) * S::TILE;
        const int k0 = jt * kBK;
        const bool more = jt + 1 < nkt;
        if (more) {
            kc.load(Kh, k0 + kBK, N, tid);
            vc.load(Vh, k0 + kBK, N, tid);
        }
        const bool active = !CAUSAL || k0 <= wq0 + kRowsPerWave - 1;
        if (active) {
            // ---- S^T = K Q^T for the 64 keys of the tile (two 32-key blocks)
            f32x16 s[S::KB];
#pragma unroll
            for (int kb = 0; kb < S::KB; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
                const uint16_t* kp = Ks + buf + (kb * 32 + n32) * S::STR + 8 * h;
#pragma unroll
                for (int ks = 0; ks < S::KS; ++ks)
                    s[kb] = mfma32<T>(*(const u32x4*)(kp + 16 * ks), qf[ks], s[kb]);
            }
            // ---- mask the diagonal tile and the ragged end of the sequence
            const bool masked = (k0 + kBK > N) || (CAUSAL && k0 + kBK - 1 > wq0);
            if (masked) {
#pragma unroll
                for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key >= N || (CAUSAL && key > qrow)) s[kb][e] = kNegInf;
                    }
            }
            // ---- online softmax: raise the maximum, rescale when it grew
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
            mx = max_with_other_half(mx);
            const float mnew = fmaxf(m, mx);
            if (__any(mnew > m)) {
                const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < S::DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            }
            m = mnew;
            const float mc = (m == kNegInf) ? 0.f : m * c;
            // ---- P^T = exp2(c*s - c*m), packed as the B operand of O^T += V^T P^T
            u32x4 pf[S::KB][2];
#pragma unroll
            for (int kb = 0; kb < S::KB; ++kb) {
                f32x16 p;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c, -mc));
                    if (masked) pe = s[kb][e] == kNegInf ? 0.f : pe;
                    l += pe;
                    p[e] = pe;
                }
                pack_acc_as_b<T>(p, pf[kb][0], pf[kb][1]);
            }
            // ---- O^T += V^T P^T
            const uint16_t* vp = Vs + buf + tr_off;
#pragma unroll
            for (int db = 0; db < S::DB; ++db)
#pragma unroll
                for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        oacc[db] = mfma32<T>(tr_operand<S::STR>(vp, kb * 32 + 16 * t, 32 * db), pf[kb][t], oacc[db]);
        }
        if (more) {
            kc.store(Ks + S::TILE - buf, tid);
            vc.store(Vs + S::TILE - buf, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, staged through LDS for row-contiguous stores
    const float lt = sum_with_other_half(l);
    const float inv = 1.f / lt;
    if (h == 0 && qrow < N) LSE[(int64_t)bh * N + qrow] = m * scale + logf(lt);
    uint16_t* Os = Ks;  // the loop ended on a barrier: both K buffers are free
    const int orow = (w * kRowsPerWave + n32) * S::STR;
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 pk = {pack2<T>(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                        pack2<T>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
            *(u32x2*)(Os + orow + 32 * db + 8 * g + 4 * h) = pk;
        }
    __syncthreads();
    uint16_t* Oh = O + base;
    for (int ch = tid; ch < kBQ * S::CH; ch += kThreads) {
        const int r = ch / S::CH, col = ch % S::CH;
        if (q0 + r < N) *(u32x4*)(Oh + (int64_t)(q0 + r) * D + 8 * col) = *(const u32x4*)(Os + r * S::STR + 8 * col);
    }
}

template <class T, int D, bool CAUSAL>
hipError_t launch(const FwdParams& p) {
    const int ntq = (p.N + kBQ - 1) / kBQ;
    const int64_t blocks = (int64_t)p.B * p.H * ntq;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                       (const uint16_t*)p.v, (uint16_t*)p.o, p.lse, p.N, ntq, p.scale,
                       p.scale * kLog2e);
    return hipGetLastError();
}

template <class T, int D>
hipError_t launch_c(const FwdParams& p) {
    return p.causal ? launch<T, D, true>(p) : launch<T, D, false>(p);
}

template <class T>
hipError_t launch_d(const FwdParams& p) {
    return p.d == 64 ? launch_c<T, 64>(p) : launch_c<T, 128>(p);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p) {
    return p.dtype == kDtypeBF16 ? launch_d<BF16>(p) : launch_d<F16>(p);
}

}  // namespace attn
