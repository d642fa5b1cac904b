// attn_bwd.hip -- recompute backward of fused exact attention for gfx950.
//
// Only O and the per-row lse were kept by the forward; the score tiles are
// rebuilt here from Q, K and lse (the hotdry blog's section "4. 重计算
// （Recomputation）策略": store one statistic per row, recompute the QK^T
// blocks in the backward pass, stream the gradients).  With
// P = exp(scale * Q K^T - lse) (zero where masked) and D_i = <dO_i, O_i>:
//
//     dV = P^T dO,   dS = P o (dO V^T - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Two kernels, neither with atomics (fp32 global atomics run at ~1.3 TB/s on
// this part, far too slow for per-tile dQ partial sums):
//
//   attn_bwd_dq_kernel    query-tile stationary.  Computes D for its rows
//                         (written to the workspace), then streams K and V
//                         tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, and
//                         dQ^T += K^T dS^T.  Same orientation as the forward:
//                         lane l owns query l % 32, so lse and D are per-lane
//                         scalars.
//   attn_bwd_dkdv_kernel  key-tile stationary, launched second (it reads D).
//                         K and V of its 128 keys stay in registers; it
//                         streams Q and dO tiles: S = Q K^T, dP = dO V^T,
//                         dV^T += dO^T P, dK^T += Q^T dS.  Here lane l owns
//                         key l % 32, so P and dS leave their accumulators
//                         directly as B operands.
//
// The second kernel recomputes S and dP, so the backward performs seven
// d-deep products per unmasked pair instead of five; it buys freedom from
// atomics and a deterministic result.
//
// Both kernels stream their tiles through LDS by DMA (in the swizzled layout
// of DmaTile: double-buffered in the first, a ring of three in the second,
// which overlaps the vector work of one query block with the matrix products
// of the block before) and, with a block mask, visit only the tiles of active
// (query block, key block) pairs.

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr float kPosInf = __builtin_inff();

// 16-bit storage -> fp32.
template <class T>
__device__ inline float lo16(uint32_t u);
template <class T>
__device__ inline float hi16(uint32_t u);
template <>
__device__ inline float lo16<BF16>(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
template <>
__device__ inline float hi16<BF16>(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
template <>
__device__ inline float lo16<F16>(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
}
template <>
__device__ inline float hi16<F16>(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

template <class T>
__device__ inline float dot8(const u32x4& a, const u32x4& b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += lo16<T>(a[i]) * lo16<T>(b[i]) + hi16<T>(a[i]) * hi16<T>(b[i]);
    return s;
}

// Write a wave's 32 x D accumulator tile (lane l: column l % 32 of each 32-row
// block db, rows 32*db + 8*(e/4) + 4*(l/32) + e%4), times `mul`, transposed
// into row (row0 + l % 32) of a row-major LDS staging tile.
template <class T, int D, int STR>
__device__ inline void stage_transposed(uint16_t* st, int row, int h, const f32x16 (&acc)[D / 32], float mul) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 pk = {pack2<T>(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                        pack2<T>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
            *(u32x2*)(st + row * STR + 32 * db + 8 * g + 4 * h) = pk;
        }
}

// Copy `rows` staged rows (row r of the tile -> global row r0 + r, if < N).
template <int D, int STR>
__device__ inline void store_staged(uint16_t* __restrict__ dst, const uint16_t* st, int rows, int r0, int N, int tid) {
    constexpr int CH = D / 8;
    for (int ch = tid; ch < rows * CH; ch += kThreads) {
        const int r = ch / CH, col = ch % CH;
        if (r0 + r < N) *(u32x4*)(dst + (int64_t)(r0 + r) * D + 8 * col) = *(const u32x4*)(st + r * STR + 8 * col);
    }
}

// ============================================================================
// dQ and D: one work group per (sequence, 128 query rows), 4 waves x 32 rows.
// K and V tiles of 64 keys stream through LDS by DMA (double-buffered).
// ============================================================================
constexpr int kQ_BQ = 128;
constexpr int kQ_BK = 64;

// Runs of unmasked key tiles go through a hand-scheduled walk
// (attn_dq_loop.inc, written by gen_dq_loop.py): each accumulator sees the
// operands and order of the step below, so bitwise-equal results, with the
// exponentials and dS of each key block issued between the MFMAs as soon as
// their inputs exist.  ATTN_DQ_ASM=0 builds the kernel with the C++ step only.
#ifndef ATTN_DQ_ASM
#define ATTN_DQ_ASM 1
#endif
#if ATTN_DQ_ASM
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#include "attn_dq_loop.inc"
#pragma clang diagnostic pop
#endif

template <class T, int D, bool BS>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
                        const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
                        float* __restrict__ Delta, uint16_t* __restrict__ dQ, SeqLayout L, int ntq,
                        float scale, float c) {
    using DT = DmaTile<D, kQ_BK>;
    constexpr int STR = LdsStride<D>::value;  // row stride of the output staging
    constexpr int KS = D / 16, DB = D / 32, KB = kQ_BK / 32;
    constexpr int TB = DT::ELEMS;
    constexpr int SMEM = (kQ_BQ * STR > 4 * TB) ? kQ_BQ * STR : 4 * TB;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM];
    uint16_t* const Ks = smem;           // K tiles: buffers 0, 1
    uint16_t* const Vs = smem + 2 * TB;  // V tiles: buffers 0, 1

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const Seq sq = resolve(L, item / ntq);
    const int qt = (L.wr >= 0 && L.wl < 0) ? ntq - 1 - item % ntq : item % ntq;
    const int q0 = qt * kQ_BQ;
    if (q0 >= sq.nq) return;  // the whole group: no barrier has been reached
    const int nq = sq.nq, nk = sq.nk;
    const uint16_t *Qh = Q + sq.qrow0 * D, *Oh = O + sq.qrow0 * D, *dOh = dO + sq.qrow0 * D;
    const uint16_t *Kh = K + sq.krow0 * D, *Vh = V + sq.krow0 * D;
    const int wq0 = q0 + 32 * w;
    const int qrow = wq0 + n32;
    const bool valid = qrow < nq;

    // Resident Q^T and dO^T fragments; D = <dO, O> for this row.  Rows past
    // the end read row nq-1: their D is not stored, their lse is +inf (P = 0),
    // and their dQ is not written.
    u32x4 qf[KS], dof[KS];
    float dpart = 0.f;
    const int qrd = min(qrow, nq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int64_t off = (int64_t)qrd * D + 16 * ks + 8 * h;
        qf[ks] = *(const u32x4*)(Qh + off);
        dof[ks] = *(const u32x4*)(dOh + off);
        const u32x4 of = *(const u32x4*)(Oh + off);
        dpart += dot8<T>(dof[ks], of);
    }
    const float Dq = sum_with_other_half(dpart);
    // stored negated: the dK/dV kernel starts its dP accumulators from -D
    if (h == 0 && valid) Delta[sq.qrow0 + qrow] = -Dq;
    const float lse2 = valid ? LSE[sq.qrow0 + qrd] * kLog2e : kPosInf;

    // Key tiles some row of the group sees, and those every row sees in full.
    const int qlast = min(q0 + kQ_BQ, nq) - 1;
    const TileRange tr = tile_range(sq.key_lo(q0), sq.key_hi(qlast), sq.key_lo(qlast),
                                    min(sq.key_hi(q0), nk - 1), nk, kQ_BK);
    const uint32_t goff = DT::lane_goff(lane);
    // With a block mask only the key tiles of active (query block, key block)
    // pairs are visited (a 64-key tile lies in mask block t / 2; the mask is
    // read with uniform loads).
    static_assert(!BS || (kQ_BQ == kMaskBlock && 2 * kQ_BK == kMaskBlock), "block masks need 128-row groups");
    const uint8_t* bmrow = BS ? sq.bm + (size_t)(q0 / kMaskBlock) * sq.nb : nullptr;
    auto next_tile = [&](int t) __attribute__((always_inline)) {
        ++t;
        if (BS)
            while (t < tr.end && !bmrow[t >> 1]) ++t;
        return t;
    };
    int j0 = tr.first;
    if (BS)
        while (j0 < tr.end && !bmrow[j0 >> 1]) ++j0;
    if (j0 < tr.end) {
        dma_tile<D, kQ_BK>(Kh, j0 * kQ_BK, nk, Ks, w, lane, goff);
        dma_tile<D, kQ_BK>(Vh, j0 * kQ_BK, nk, Vs, w, lane, goff);
    }
    // Unconditional: the fragments above and the first tiles have landed (the
    // compiler counts only its own loads; see the forward kernel).
    wait_dma();
    __syncthreads();

    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dqacc[db][e] = 0.f;
    const uint32_t fo[2] = {DT::frag_lane(lane, 0), DT::frag_lane(lane, 1)};
    const uint32_t to0 = DT::tr_lane(lane, 0), to1 = DT::tr_lane(lane, 1);

    // Tile jt in buffer buf; jn is the next tile visited.
    auto step = [&](int jt, int jn, int buf, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int k0 = jt * kQ_BK;
        // the other buffers held the previous tile, which every wave has finished
        if (jn < tr.end) {
            dma_tile<D, kQ_BK>(Kh, jn * kQ_BK, nk, Ks + (1 - buf) * TB, w, lane, goff);
            dma_tile<D, kQ_BK>(Vh, jn * kQ_BK, nk, Vs + (1 - buf) * TB, w, lane, goff);
        }
        if (!MASKED || (wq0 < nq && k0 <= sq.key_hi(wq0 + 31) && k0 + kQ_BK - 1 >= sq.key_lo(wq0))) {
            const char* kt = (const char*)(Ks + buf * TB);
            const char* vt = (const char*)(Vs + buf * TB);
            // ---- S^T = K Q^T and dP^T = V dO^T
            f32x16 s[KB], dp[KB];
            prio_mfma();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    s[kb][e] = 0.f;
                    dp[kb][e] = -Dq;  // dP^T starts from -D: the products leave dP^T - D
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int o = DT::frag_blk(kb, ks);
                    s[kb] = mfma32<T>(*(const u32x4*)(kt + fo[ks & 1] + o), qf[ks], s[kb]);
                    dp[kb] = mfma32<T>(*(const u32x4*)(vt + fo[ks & 1] + o), dof[ks], dp[kb]);
                }
            }
            sched_reads_ahead<4, 2 * KB * KS, 1>();
            prio_normal();
            // ---- P^T = exp(scale s - lse), dS^T = P^T o (dP^T - D), dP^T - D already in dp
            const int klo = sq.key_lo(qrow), khi = min(sq.key_hi(qrow), nk - 1);
            u32x4 b[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16 ds;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c, -lse2));
                    if constexpr (MASKED) {
                        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key < klo || key > khi) p = 0.f;
                    }
                    ds[e] = p * dp[kb][e];
                }
                pack_acc_as_b<T>(ds, b[kb][0], b[kb][1]);
            }
            // ---- dQ^T += K^T dS^T (K^T read transposed from the K tile)
            prio_mfma();
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        dqacc[db] = mfma32<T>(tr_operand_dma(kt, to0, to1, DT::tr_blk(2 * kb + t, db)), b[kb][t],
                                              dqacc[db]);
            sched_reads_ahead<8, DB * KB * 2, 2>();
            prio_normal();
        }
        wait_dma();
        __syncthreads();
    };
    if constexpr (!BS) {
        for (int jt = tr.first; jt < tr.full_first; ++jt) step(jt, jt + 1, jt - tr.first & 1, Flag<true>{});
        int ua = tr.full_first;
#if ATTN_DQ_ASM
        {
            // Tiles [ua, bb) through the hand-scheduled walk: unmasked, each
            // loading a whole next tile (jt + 1 < tr.end, ending within nk).
            // It enters after a step's barrier (tile ua landed, nothing in
            // flight) and leaves in the same state for tile bb.
            const int bb = min(tr.full_end, min(tr.end, nk / kQ_BK) - 1);
            if (bb > ua) {
                const uint32_t sm = lds_addr(smem);
                const uint32_t mk0 = __builtin_amdgcn_readfirstlane(sm + w * 1024);
                const uint32_t mv0 = mk0 + 2 * DT::BYTES;
                const int rg = w / DT::CG, cg = w % DT::CG;
                const uint64_t wofs = (uint64_t)((rg * 16 * D + cg * 32) * 2);
                // readfirstlane returns a signed int: each half goes through uint32_t
                auto uniform64 = [](uint64_t x) __attribute__((always_inline)) {
                    return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32);
                };
                const uint64_t t1 = (uint64_t)(ua + 1);
                const uint64_t ksrc = uniform64((uint64_t)(uintptr_t)Kh + t1 * DT::BYTES + wofs);
                const uint64_t vsrc = uniform64((uint64_t)(uintptr_t)Vh + t1 * DT::BYTES + wofs);
                dq_unmasked_run<T, D>(dqacc, qf, dof, lse2, Dq, sm + fo[0], sm + fo[1], sm + to0, sm + to1, goff, c,
                                      (uint32_t)((ua - tr.first) & 1), mk0, mk0 + DT::BYTES, mv0, mv0 + DT::BYTES,
                                      ksrc, vsrc, (uint32_t)(bb - ua));
                ua = bb;
            }
        }
#endif
        for (int jt = ua; jt < tr.full_end; ++jt) step(jt, jt + 1, jt - tr.first & 1, Flag<false>{});
        for (int jt = tr.full_end; jt < tr.end; ++jt) step(jt, jt + 1, jt - tr.first & 1, Flag<true>{});
    } else {
        // The visited tiles ascend; masked ones lie before full_first or from
        // full_end on.  One loop per kind: a loop whose body branched between
        // the kinds would have the compiler copy the accumulators every tile.
        int jt = j0, buf = 0;
        auto run = [&](int lim, auto masked_tag) __attribute__((always_inline)) {
            while (jt < lim) {
                const int jn = next_tile(jt);
                step(jt, jn, buf, masked_tag);
                jt = jn;
                buf ^= 1;
            }
        };
        run(tr.full_first, Flag<true>{});
        run(tr.full_end, Flag<false>{});
        run(tr.end, Flag<true>{});
    }

    stage_transposed<T, D, STR>(smem, 32 * w + n32, h, dqacc, scale);
    __syncthreads();
    store_staged<D, STR>(dQ + sq.qrow0 * D, smem, kQ_BQ, q0, nq, tid);
}

// ============================================================================
// dK and dV: one work group per (sequence, 128 key rows), 4 waves x 32 keys.
// Q and dO tiles of 64 rows stream through LDS by DMA, in a ring of three
// buffers.
//
// Software pipeline (per wave, over the 32-row query blocks b of the visited
// tiles): while the vector unit forms P and dS of block b, the matrix cores
// run the dV, dK products of block b - 1.  With one wave per SIMD (d = 128)
// no other wave could fill the matrix cores while this one does vector work,
// so the overlap has to come from independent instructions of the same wave.
// Block b - 1 may lie in the previous tile, which therefore stays in LDS
// while the tile after the current one is loaded: a ring of three.
// ============================================================================
constexpr int kK_BK = 128;
constexpr int kK_BQ = 64;
constexpr int kK_NBUF = 3;

// Runs of unmasked query tiles at d = 128 go through a hand-scheduled walk
// (attn_dkdv_loop.inc, written by gen_dkdv_loop.py): the instructions and
// accumulation order of the tile below, so bitwise-equal results, with the
// vector work of each block spread over two MFMA runs and LDS operands read
// well ahead.  ATTN_DKDV_ASM=0 builds the kernel with the C++ tile only.
#ifndef ATTN_DKDV_ASM
#define ATTN_DKDV_ASM 1
#endif
#if ATTN_DKDV_ASM
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#include "attn_dkdv_loop.inc"
#pragma clang diagnostic pop
#endif

template <class T, int D, bool BS>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(D == 64 ? 2 : 1, 2)))
void attn_bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Delta,
                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, SeqLayout L, int ntk,
                          float scale, float c) {
    using DT = DmaTile<D, kK_BQ>;
    constexpr int STR = LdsStride<D>::value;  // row stride of the output staging
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TB = DT::ELEMS;
    constexpr int SMEM = (kK_BK * STR > 2 * kK_NBUF * TB) ? kK_BK * STR : 2 * kK_NBUF * TB;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM];  // buffer b: Q tile 2b, dO tile 2b + 1
    __shared__ __attribute__((aligned(16))) float stats[kK_NBUF][2][kK_BQ];  // [buffer][lse*log2e, -D][row]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const Seq sq = resolve(L, item / ntk);
    const int kt = item % ntk;  // causal: low key tiles see the most queries and run first
    const int k0 = kt * kK_BK;
    if (k0 >= sq.nk) return;  // the whole group: no barrier has been reached
    const int nq = sq.nq, nk = sq.nk;
    const uint16_t *Qh = Q + sq.qrow0 * D, *dOh = dO + sq.qrow0 * D;
    const uint16_t *Kh = K + sq.krow0 * D, *Vh = V + sq.krow0 * D;
    const float* lseh = LSE + sq.qrow0;
    const float* Dh = Delta + sq.qrow0;  // -D of each row, as the dq kernel stores it
    const int krow = k0 + 32 * w + n32;

    // Resident K and V fragments (B operands of S = Q K^T and dP = dO V^T).
    // Keys past the end read row nk-1; their dK and dV are never written.
    u32x4 kf[KS], vf[KS];
    const int krd = min(krow, nk - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int64_t off = (int64_t)krd * D + 16 * ks + 8 * h;
        kf[ks] = *(const u32x4*)(Kh + off);
        vf[ks] = *(const u32x4*)(Vh + off);
    }

    // Query tiles in which some row sees a key of the group, and those whose
    // every row sees every key of the group (rows past the end need no mask:
    // their lse is +inf, so P = 0).
    const int klast = min(k0 + kK_BK, nk) - 1;
    const TileRange tr = tile_range(sq.row_lo(k0), sq.row_hi(klast), sq.row_lo(klast), sq.row_hi(k0), nq, kK_BQ);
    const uint32_t goff = DT::lane_goff(lane);
    // With a block mask only the query tiles of active (query block, key
    // block) pairs are visited: a 64-row tile lies in mask block t / 2, and
    // this group's 128 keys are key block kt (the mask column is read with
    // uniform loads).
    static_assert(!BS || (kK_BK == kMaskBlock && 2 * kK_BQ == kMaskBlock), "block masks need 128-key groups");
    const uint8_t* bmcol = BS ? sq.bm + kt : nullptr;
    auto next_tile = [&](int t) __attribute__((always_inline)) {
        ++t;
        if (BS)
            while (t < tr.end && !bmcol[(size_t)(t >> 1) * sq.nb]) ++t;
        return t;
    };

    // Tile `it` into ring buffer b: Q and dO by DMA, the row statistics into
    // registers (stored to LDS later, once the buffer's previous statistics
    // are no longer read; lse is scaled by log2(e) as it is stored).
    float st_l = kPosInf, st_d = 0.f;
    auto fetch = [&](int it, int b) __attribute__((always_inline)) {
        const int r0 = it * kK_BQ;
        dma_tile<D, kK_BQ>(Qh, r0, nq, smem + 2 * b * TB, w, lane, goff);
        dma_tile<D, kK_BQ>(dOh, r0, nq, smem + (2 * b + 1) * TB, w, lane, goff);
        if (tid < kK_BQ) {
            const int r = r0 + tid;
            st_l = r < nq ? lseh[r] : kPosInf;  // rows past the end get P = 0
            st_d = r < nq ? Dh[r] : 0.f;
        }
    };
    auto store_stats = [&](int b) __attribute__((always_inline)) {
        if (tid < kK_BQ) {
            stats[b][0][tid] = st_l * kLog2e;
            stats[b][1][tid] = st_d;
        }
    };

    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            dkacc[db][e] = 0.f;
            dvacc[db][e] = 0.f;
        }
    const uint32_t fo[2] = {DT::frag_lane(lane, 0), DT::frag_lane(lane, 1)};
    const uint32_t to0 = DT::tr_lane(lane, 0), to1 = DT::tr_lane(lane, 1);

    // ---- the parts of a block (qb: the block's index in its tile).  Each
    // issues all LDS operand reads of its MFMAs first, then runs as a fixed
    // sequence of steps, one MFMA per step; a scheduling barrier after every
    // step keeps the compiler from regrouping the vector work (measured: one
    // element's vector work per MFMA step is fastest at d = 128).
    // S = Q K^T and dP = dO V^T of block qb of the tile in buffer b.
    // Operand i: k-step i / 2 of S (i even, Q fragment) or dP (i odd, dO).
    auto part_a = [&](int b, auto qb_tag, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
        constexpr int QBI = decltype(qb_tag)::value;
        const char* qt_ = (const char*)(smem + 2 * b * TB);
        const char* ot_ = (const char*)(smem + (2 * b + 1) * TB);
        auto rd = [&](int i) __attribute__((always_inline)) {
            return *(const u32x4*)(((i & 1) ? ot_ : qt_) + fo[(i >> 1) & 1] + DT::frag_blk(QBI, i >> 1));
        };
        u32x4 fa[2 * KS];
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) fa[i] = rd(i);
        // dP starts from -D of the rows this lane holds (8g + 4h + 0..3), so
        // the products leave dP - D, the factor of dS, in the accumulator
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 nd = *(const f32x4*)(&stats[b][1][32 * QBI + 8 * g + 4 * h]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[4 * g + r] = 0.f;
                dp[4 * g + r] = nd[r];
            }
        }
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
            if (i & 1) dp = mfma32<T>(fa[i], vf[i >> 1], dp);
            else s = mfma32<T>(fa[i], kf[i >> 1], s);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // dV^T += dO^T P and dK^T += Q^T dS of a previous block (qb QP, buffer bq;
    // skipped when PREV is false), interleaved with P = exp(scale s - lse),
    // dS = P o (dP - D) of the current block (qb QC, first row qb0, statistics
    // in buffer b), packed as B operands.  MFMA i: 32-row block i / 4 of d,
    // k-half (i / 2) % 2, dV (i even, dO^T read transposed) or dK (i odd,
    // Q^T); vector step e: element e of the current block.
    auto part_bv = [&](auto prev_tag, int bq, auto qp_tag, const u32x4 (&bpp)[2], const u32x4 (&bdp)[2], int b, int qb0,
                       auto qc_tag, auto masked_tag, const f32x16& s, const f32x16& dp, u32x4 (&bpo)[2],
                       u32x4 (&bdo)[2]) __attribute__((always_inline)) {
        constexpr bool PREV = decltype(prev_tag)::value;
        constexpr int QP = decltype(qp_tag)::value;
        constexpr int QC = decltype(qc_tag)::value;
        constexpr bool MASKED = decltype(masked_tag)::value;
        constexpr int NB = 4 * DB;  // MFMAs of the previous block: one every 16 / NB elements
        const char* qt_ = (const char*)(smem + 2 * bq * TB);
        const char* ot_ = (const char*)(smem + (2 * bq + 1) * TB);
        auto rd = [&](int i) __attribute__((always_inline)) {
            return tr_operand_dma((i & 1) ? qt_ : ot_, to0, to1, DT::tr_blk(2 * QP + ((i >> 1) & 1), i >> 2));
        };
        // lse * log2(e) of the query rows this lane holds: 8g + 4h + (0..3)
        f32x4 l4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) l4[g] = *(const f32x4*)(&stats[b][0][32 * QC + 8 * g + 4 * h]);
        u32x4 ta[NB];
        if (PREV) {
#pragma unroll
            for (int i = 0; i < NB; ++i) ta[i] = rd(i);
        }
        float pv[16], dv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (PREV && (e * NB) % 16 == 0) {
                const int i = e * NB / 16;
                if (i & 1) dkacc[i >> 2] = mfma32<T>(ta[i], bdp[(i >> 1) & 1], dkacc[i >> 2]);
                else dvacc[i >> 2] = mfma32<T>(ta[i], bpp[(i >> 1) & 1], dvacc[i >> 2]);
            }
            const int g = e >> 2, r = e & 3;
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, -l4[g][r]));
            if constexpr (MASKED) {
                if (!sq.visible(qb0 + 8 * g + 4 * h + r, krow)) pe = 0.f;
            }
            pv[e] = pe;
            dv[e] = pe * dp[e];  // dp holds dP - D (part_a)
            if (e & 1) {
                bpo[e >> 3][(e & 7) >> 1] = pack2<T>(pv[e - 1], pv[e]);
                bdo[e >> 3][(e & 7) >> 1] = pack2<T>(dv[e - 1], dv[e]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Pin the packed results here: they are used only by the next
        // block's products, and the compiler would otherwise sink this whole
        // vector computation past the tile barrier, out of the MFMA shadow.
        asm volatile("" : "+v"(bpo[0]), "+v"(bpo[1]), "+v"(bdo[0]), "+v"(bdo[1]));
    };
    // dV, dK products alone (the walk's last block).
    auto part_b = [&](int bq, auto qp_tag, const u32x4 (&bpp)[2], const u32x4 (&bdp)[2]) __attribute__((always_inline)) {
        constexpr int QP = decltype(qp_tag)::value;
        const char* qt_ = (const char*)(smem + 2 * bq * TB);
        const char* ot_ = (const char*)(smem + (2 * bq + 1) * TB);
#pragma unroll
        for (int i = 0; i < 4 * DB; ++i) {
            const u32x4 a = tr_operand_dma((i & 1) ? qt_ : ot_, to0, to1, DT::tr_blk(2 * QP + ((i >> 1) & 1), i >> 2));
            if (i & 1) dkacc[i >> 2] = mfma32<T>(a, bdp[(i >> 1) & 1], dkacc[i >> 2]);
            else dvacc[i >> 2] = mfma32<T>(a, bpp[(i >> 1) & 1], dvacc[i >> 2]);
        }
    };

    // Per-wave pipeline registers: S, dP of the current block; packed P, dS
    // of the blocks with index 0 / 1 in their tile.
    f32x16 sc, dpc;
    u32x4 bp[2][2], bds[2][2];

    // Walk state: tiles it (position n in the walk, ring buffer bc), in1 and
    // in2 (the next two); bn and bpv are the buffers of positions n + 1 and
    // n - 1 (== n + 2).
    int it = tr.first;
    if (BS)
        while (it < tr.end && !bmcol[(size_t)(it >> 1) * sq.nb]) ++it;
    int in1 = it < tr.end ? next_tile(it) : tr.end;
    int in2 = in1 < tr.end ? next_tile(in1) : tr.end;
    int bc = 0, bn = 1, bpv = 2;
    if (it < tr.end) {
        fetch(it, 0);
        store_stats(0);
        if (in1 < tr.end) fetch(in1, 1);  // its statistics are stored at the first tile boundary
    }
    wait_dma();  // unconditional (see the dq kernel)
    __syncthreads();
    if (it < tr.end) {
        // One tile: for each of its two blocks, S and dP on the matrix cores,
        // then P and dS on the vector unit while the matrix cores run the dV,
        // dK products of the block before (FIRST: the walk's first tile has
        // none before its block 0).
        auto tile = [&](auto masked_tag, auto first_tag) __attribute__((always_inline)) {
            constexpr bool FIRST = decltype(first_tag)::value;
            const int qq0 = it * kK_BQ;
            prio_mfma();
            part_a(bc, Flag<0>{}, sc, dpc);
            part_bv(Flag<!FIRST>{}, bpv, Flag<1>{}, bp[1], bds[1], bc, qq0, Flag<0>{}, masked_tag, sc, dpc, bp[0], bds[0]);
            part_a(bc, Flag<1>{}, sc, dpc);
            part_bv(Flag<true>{}, bc, Flag<0>{}, bp[0], bds[0], bc, qq0 + 32, Flag<1>{}, masked_tag, sc, dpc, bp[1], bds[1]);
            prio_normal();
        };
        // Tile boundary: every wave has finished tile it and the previous
        // one (apart from block 1 of tile it, whose dV, dK products run with
        // the next tile), the DMA of tile in1 has landed, and tile in2 goes
        // into the buffer of the previous tile.
        auto boundary = [&]() __attribute__((always_inline)) {
            wait_dma();
            if (in1 < tr.end) store_stats(bn);
            __syncthreads();
            if (in2 < tr.end) fetch(in2, bpv);
            it = in1;
            in1 = in2;
            in2 = in2 < tr.end ? next_tile(in2) : tr.end;
            const int b0 = bpv;
            bpv = bc;
            bc = bn;
            bn = b0;
        };
        auto masked_tile = [&](int t) { return t < tr.full_first || t >= tr.full_end; };

        if (masked_tile(it)) tile(Flag<true>{}, Flag<true>{});
        else tile(Flag<false>{}, Flag<true>{});
        boundary();
        // The visited tiles ascend, and the masked ones lie before full_first
        // or from full_end on: one loop per kind, so that each loop body has
        // a single register assignment (a loop whose body branches between
        // the two kinds has the compiler copy the accumulators every tile).
        auto run = [&](int lim, auto masked_tag) __attribute__((always_inline)) {
            while (it < lim) {
                tile(masked_tag, Flag<false>{});
                boundary();
            }
        };
        run(tr.full_first, Flag<true>{});
#if ATTN_DKDV_ASM
        if constexpr (D == 128 && !BS) {
            // Tiles [it, bb) through the hand-scheduled walk: unmasked, not the
            // walk's first, and every boundary fetching a whole tile (it + 2 <
            // tr.end, ending within nq).  Entry and exit are at a tile start,
            // with the state the C++ tile and boundary leave there.
            const int bb = min(tr.full_end, min(tr.end, nq / kK_BQ) - 2);
            if (bb > it) {
                const uint32_t sm = lds_addr(smem);
                const uint32_t hi = 3 * DT::BYTES;
                const uint32_t f4[4] = {sm + fo[0], sm + fo[1], sm + fo[0] + hi, sm + fo[1] + hi};
                const uint32_t t4[4] = {sm + to0, sm + to1, sm + to0 + hi, sm + to1 + hi};
                const uint32_t sta = lds_addr(&stats[0][0][0]);
                const uint32_t g4[4] = {goff, goff + 4096, goff + 8192, goff + 12288};
                const uint32_t mw = __builtin_amdgcn_readfirstlane(sm + w * 1024);
                const uint32_t mq[3] = {mw, mw + 2 * DT::BYTES, mw + 4 * DT::BYTES};
                const uint32_t md[3] = {mw + DT::BYTES, mw + 3 * DT::BYTES, mw + 5 * DT::BYTES};
                const int rg = w / DT::CG, cg = w % DT::CG;
                const uint64_t wofs = (uint64_t)((rg * 16 * D + cg * 32) * 2);
                // readfirstlane returns a signed int: each half goes through uint32_t
                auto uniform64 = [](uint64_t x) __attribute__((always_inline)) {
                    return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32);
                };
                const uint64_t t2 = (uint64_t)(it + 2);
                const uint64_t qsrc = uniform64((uint64_t)(uintptr_t)Qh + t2 * DT::BYTES + wofs);
                const uint64_t dosrc = uniform64((uint64_t)(uintptr_t)dOh + t2 * DT::BYTES + wofs);
                const uint64_t lsrc = uniform64((uint64_t)(uintptr_t)lseh + t2 * kK_BQ * 4);
                const uint64_t dsrc = uniform64((uint64_t)(uintptr_t)Dh + t2 * kK_BQ * 4);
                const int n = bb - it;
                dkdv_unmasked_run<T, D>(dvacc, dkacc, kf, vf, bp[1], bds[1], st_l, st_d, f4, t4, sta + 16 * h,
                                        sta + 4 * lane, g4, 4 * lane, c, (uint32_t)w, (uint32_t)bc, mq, md, qsrc,
                                        dosrc, lsrc, dsrc, (uint32_t)n);
                it = bb;
                in1 = bb + 1;
                in2 = min(bb + 2, tr.end);
                bc = (bc + n) % 3;
                bn = (bn + n) % 3;
                bpv = (bpv + n) % 3;
            }
        }
#endif
        run(tr.full_end, Flag<false>{});
        run(tr.end, Flag<true>{});
        // block 1 of the last tile (now the previous buffer)
        prio_mfma();
        part_b(bpv, Flag<1>{}, bp[1], bds[1]);
        prio_normal();
    }

    // the ring buffers are reused as output staging
    __syncthreads();
    stage_transposed<T, D, STR>(smem, 32 * w + n32, h, dkacc, scale);
    __syncthreads();
    store_staged<D, STR>(dK + sq.krow0 * D, smem, kK_BK, k0, nk, tid);
    __syncthreads();
    stage_transposed<T, D, STR>(smem, 32 * w + n32, h, dvacc, 1.f);
    __syncthreads();
    store_staged<D, STR>(dV + sq.krow0 * D, smem, kK_BK, k0, nk, tid);
}

template <class T, int D, bool BS>
hipError_t launch(const BwdParams& p) {
    const int ntq = (p.max_nq + kQ_BQ - 1) / kQ_BQ;
    const int ntk = (p.max_nk + kK_BK - 1) / kK_BK;
    const int64_t nseq = (int64_t)p.L.B * p.L.H;
    if (nseq * ntq > 0x7fffffff || nseq * ntk > 0x7fffffff) return hipErrorInvalidConfiguration;
    const float c = p.scale * kLog2e;
    hipStream_t st = (hipStream_t)p.stream;
    if (nseq * ntq > 0) {
        hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BS>), dim3((unsigned)(nseq * ntq)), dim3(kThreads), 0, st,
                           (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (const uint16_t*)p.o,
                           (const uint16_t*)p.dout, p.lse, p.delta, (uint16_t*)p.dq, p.L, ntq, p.scale, c);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (nseq * ntk > 0) {
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, BS>), dim3((unsigned)(nseq * ntk)), dim3(kThreads), 0, st,
                           (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (const uint16_t*)p.dout,
                           p.lse, p.delta, (uint16_t*)p.dk, (uint16_t*)p.dv, p.L, ntk, p.scale, c);
    }
    return hipGetLastError();
}

template <class T, bool BS>
hipError_t launch_d(const BwdParams& p) {
    return p.d == 64 ? launch<T, 64, BS>(p) : launch<T, 128, BS>(p);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p) {
    if (p.L.bmask) return p.dtype == kDtypeBF16 ? launch_d<BF16, true>(p) : launch_d<F16, true>(p);
    return p.dtype == kDtypeBF16 ? launch_d<BF16, false>(p) : launch_d<F16, false>(p);
}

}  // namespace attn
