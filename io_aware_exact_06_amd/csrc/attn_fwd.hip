// attn_fwd.hip -- fused exact-attention forward for gfx950.
//
// One work group owns BQ query rows of one (batch, head): four waves, each
// owning QB blocks of 32 rows.  The group streams the keys and values in
// tiles of BK = 64 rows through LDS (double-buffered; the next tile is
// prefetched into registers while the current one is consumed), and each
// wave keeps, for its rows, the running maximum m, the running sum l and the
// partial output in registers: the online softmax of the hotdry blog's
// section "3. 在线softmax算法" (initialise m = -inf and l = 0; for every key
// block raise the maximum, rescale the running sum and the partial output
// when it grew, add the block's exponentials and their weighted values).
// Only O and lse = scale * m + ln l leave the chip (section "1. 内核融合策略":
// write only the final output; section "4. 重计算" keeps one statistic per
// row).
//
// Orientation: every product is computed transposed, S^T = K Q^T and
// O^T = V^T P^T, on the 32x32x16 MFMA.  In that orientation accumulator lane
// l always belongs to query row l % 32 of its block, so the row maximum, row
// sum and rescale factor are per-lane scalars; the only cross-lane step is
// one exchange between lane l and lane l ^ 32, which hold the two halves of
// the same row.  The exponentials leave the S^T accumulator directly as the B
// operand of the P.V product (the key order inside an MFMA k-step is free, so
// the accumulator's own order is used), and V^T is read from the row-major V
// tile with the LDS transpose read.  Each K fragment and V^T fragment read
// from LDS feeds QB MFMAs (one per query block): LDS bandwidth per flop falls
// as 1/QB.
//
// Causal masking (snabindia chapter 1: the causal call skips the upper
// triangle): key tiles beyond the group's last row are never loaded; a query
// block skips a loaded tile that lies wholly above its rows; only tiles that
// cross the diagonal or the end of the sequence are masked element by element.

#include "attn_device.h"
#include "attn_launch.h"

// Query blocks (of 32 rows) per wave.  One block per wave, two waves per SIMD,
// measured fastest: with two blocks per wave (one wave per SIMD) the loop
// spills registers and loses the second wave's latency hiding.
#ifndef ATTN_FWD_QB
#define ATTN_FWD_QB 1
#endif

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBK = 64;  // key rows per tile

template <int D, int QB>
struct FwdShape {
    static constexpr int BQ = kWaves * 32 * QB;       // query rows per work group
    static constexpr int KS = D / 16;                 // MFMA k-steps of S^T over d
    static constexpr int DB = D / 32;                 // 32-row blocks of O^T
    static constexpr int KB = kBK / 32;               // 32-key blocks of a tile
    static constexpr int STR = LdsStride<D>::value;   // LDS row stride in elements
    static constexpr int CH = D / 8;                  // 16-byte chunks per row
    static constexpr int TILE = kBK * STR;            // elements per LDS tile
    static_assert(BQ * STR <= 4 * TILE, "output staging must fit in the tile buffers");
};

template <class T, int D, int QB>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
void attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, SeqLayout L, int ntq, float scale, float c) {
    using S = FwdShape<D, QB>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * S::TILE];
    uint16_t* const Ks = smem;               // two K tiles
    uint16_t* const Vs = smem + 2 * S::TILE;  // two V tiles

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n32 = lane & 31, h = lane >> 5;

    // Work item: (sequence, query tile).  Each XCD gets a contiguous range;
    // when rows see only keys up to a right bound (causal), tiles run longest
    // first.
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const Seq sq = resolve(L, item / ntq);
    const int qt = (L.wr >= 0 && L.wl < 0) ? ntq - 1 - item % ntq : item % ntq;
    const int q0 = qt * S::BQ;
    if (q0 >= sq.nq) return;  // the whole group: no barrier has been reached
    const int nq = sq.nq, nk = sq.nk;
    const uint16_t* Qh = Q + sq.qrow0 * D;
    const uint16_t* Kh = K + sq.krow0 * D;
    const uint16_t* Vh = V + sq.krow0 * D;
    const int wq0 = q0 + w * 32 * QB;  // first row of this wave; block qb starts at wq0 + 32 qb

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop.
    // Rows past the end read row nq-1; their outputs are never stored.
    u32x4 qf[QB][S::KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = min(wq0 + 32 * qb + n32, nq - 1);
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks) qf[qb][ks] = *(const u32x4*)(Qh + (int64_t)qrow * D + 16 * ks + 8 * h);
    }

    // Key tiles some row of the group sees, and those every row sees in full
    // (which run without any per-element test).
    const int qlast = min(q0 + S::BQ, nq) - 1;
    const TileRange tr = tile_range(sq.key_lo(q0), sq.key_hi(qlast), sq.key_lo(qlast),
                                    min(sq.key_hi(q0), nk - 1), nk, kBK);

    TileCopy<kBK, D, kThreads> kc(tid), vc(tid);
    if (tr.end > tr.first) {
        const int b0 = (tr.first & 1) * S::TILE;
        kc.load(Kh, tr.first * kBK, nk, tid);
        vc.load(Vh, tr.first * kBK, nk, tid);
        kc.store(Ks + b0);
        vc.store(Vs + b0);
    }
    __syncthreads();

    f32x16 oacc[QB][S::DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < S::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[qb][db][e] = 0.f;
    float m[QB], l[QB];  // running raw-score maximum; this lane's share of the running sum
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = kNegInf;
        l[qb] = 0.f;
    }

    const int tr_off = tr_lane_offset<S::STR>(lane);  // V^T read transposed from the V tile

    // One key tile.  MASKED tiles (the diagonal of a causal group, the ragged
    // end of the sequence) mask scores element by element; the others run
    // without any per-element test.
    auto step = [&](int jt, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int buf = (jt & 1) * S::TILE;
        const int k0 = jt * kBK;
        const bool more = jt + 1 < tr.end;
        if (more) {
            kc.load(Kh, k0 + kBK, nk, tid);
            vc.load(Vh, k0 + kBK, nk, tid);
        }
        // Query blocks of this wave that see at least one key of the tile.
        bool act[QB];
        bool any = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int r0 = wq0 + 32 * qb;
            act[qb] = !MASKED || (r0 < nq && k0 <= sq.key_hi(r0 + 31) && k0 + kBK - 1 >= sq.key_lo(r0));
            any = any || act[qb];
        }
        if (any) {
            // ---- S^T = K Q^T: each K fragment feeds every active query block
            f32x16 s[QB][S::KB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) s[qb][kb][e] = 0.f;
            prio_mfma();
#pragma unroll
            for (int kb = 0; kb < S::KB; ++kb) {
                const uint16_t* kp = Ks + buf + (kb * 32 + n32) * S::STR + 8 * h;
#pragma unroll
                for (int ks = 0; ks < S::KS; ++ks) {
                    const u32x4 a = *(const u32x4*)(kp + 16 * ks);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        if (act[qb]) s[qb][kb] = mfma32<T>(a, qf[qb][ks], s[qb][kb]);
                }
            }
            sched_reads_ahead<4, S::KB * S::KS * QB, 1>();
            prio_normal();
            u32x4 pf[QB][S::KB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                if (!act[qb]) continue;
                if constexpr (MASKED) {
                    // ---- mask keys past the end and keys outside the row's window
                    const int qrow = wq0 + 32 * qb + n32;
                    const int klo = sq.key_lo(qrow), khi = min(sq.key_hi(qrow), nk - 1);
#pragma unroll
                    for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                            if (key < klo || key > khi) s[qb][kb][e] = kNegInf;
                        }
                }
                // ---- online softmax: raise the maximum, rescale when it grew
                float mx = s[qb][0][0];
#pragma unroll
                for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb][kb][e]);
                mx = max_with_other_half(mx);
                const float mnew = fmaxf(m[qb], mx);
                if (__any(mnew > m[qb])) {
                    const float alpha = (m[qb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m[qb] - mnew) * c);
                    l[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < S::DB; ++db)
#pragma unroll
                        for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
                }
                m[qb] = mnew;
                const float mc = (mnew == kNegInf) ? 0.f : mnew * c;
                // ---- P^T = exp2(c*s - c*m), packed as the B operand of O^T += V^T P^T
#pragma unroll
                for (int kb = 0; kb < S::KB; ++kb) {
                    f32x16 p;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][e], c, -mc));
                        if constexpr (MASKED) pe = s[qb][kb][e] == kNegInf ? 0.f : pe;
                        l[qb] += pe;  // the running sum adds the fp32 exponentials
                        p[e] = pe;
                    }
                    pack_acc_as_b<T>(p, pf[qb][kb][0], pf[qb][kb][1]);
                }
            }
            // ---- O^T += V^T P^T: each V^T fragment feeds every active query block
            const uint16_t* vp = Vs + buf + tr_off;
            prio_mfma();
#pragma unroll
            for (int db = 0; db < S::DB; ++db)
#pragma unroll
                for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const u32x4 a = tr_operand<S::STR>(vp, kb * 32 + 16 * t, 32 * db);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            if (act[qb]) oacc[qb][db] = mfma32<T>(a, pf[qb][kb][t], oacc[qb][db]);
                    }
            sched_reads_ahead<8, S::DB * S::KB * 2 * QB, 2>();
            prio_normal();
        }
        if (more) {
            kc.store(Ks + S::TILE - buf);
            vc.store(Vs + S::TILE - buf);
        }
        __syncthreads();
    };
    for (int jt = tr.first; jt < tr.full_first; ++jt) step(jt, Flag<true>{});
    for (int jt = tr.full_first; jt < tr.full_end; ++jt) step(jt, Flag<false>{});
    for (int jt = tr.full_end; jt < tr.end; ++jt) step(jt, Flag<true>{});

    // ---- epilogue: O = O^T / l, staged through LDS for row-contiguous stores
    uint16_t* Os = smem;  // the loop ended on a barrier: every tile buffer is free
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wq0 + 32 * qb + n32;
        const float lt = sum_with_other_half(l[qb]);
        // a row that sees no key at all: O = 0, lse = -inf
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (h == 0 && qrow < nq) LSE[sq.qrow0 + qrow] = lt > 0.f ? m[qb] * scale + logf(lt) : kNegInf;
        const int orow = (w * 32 * QB + 32 * qb + n32) * S::STR;
#pragma unroll
        for (int db = 0; db < S::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 pk = {pack2<T>(oacc[qb][db][4 * g] * inv, oacc[qb][db][4 * g + 1] * inv),
                            pack2<T>(oacc[qb][db][4 * g + 2] * inv, oacc[qb][db][4 * g + 3] * inv)};
                *(u32x2*)(Os + orow + 32 * db + 8 * g + 4 * h) = pk;
            }
    }
    __syncthreads();
    uint16_t* Oh = O + sq.qrow0 * D;
    for (int ch = tid; ch < S::BQ * S::CH; ch += kThreads) {
        const int r = ch / S::CH, col = ch % S::CH;
        if (q0 + r < nq) *(u32x4*)(Oh + (int64_t)(q0 + r) * D + 8 * col) = *(const u32x4*)(Os + r * S::STR + 8 * col);
    }
}

template <class T, int D, int QB>
hipError_t launch_qb(const FwdParams& p) {
    using S = FwdShape<D, QB>;
    const int ntq = (p.max_nq + S::BQ - 1) / S::BQ;
    const int64_t nseq = (int64_t)p.L.B * p.L.H;
    const int64_t blocks = nseq * ntq;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, QB>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                       (const uint16_t*)p.v, (uint16_t*)p.o, p.lse, p.L, ntq, p.scale,
                       p.scale * kLog2e);
    return hipGetLastError();
}

template <class T>
hipError_t launch_d(const FwdParams& p) {
    return p.d == 64 ? launch_qb<T, 64, ATTN_FWD_QB>(p) : launch_qb<T, 128, ATTN_FWD_QB>(p);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p) {
    return p.dtype == kDtypeBF16 ? launch_d<BF16>(p) : launch_d<F16>(p);
}

}  // namespace attn
