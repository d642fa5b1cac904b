// attn_fwd.hip -- fused exact-attention forward for gfx950.
//
// One work group owns 128 query rows of one sequence (of one head): four
// waves of 32 rows (QB blocks of 32 rows per wave in general).  Keys and
// values stream through LDS in tiles of 64 rows, double-buffered and loaded
// by the DMA path (global_load_lds: global memory straight into LDS, no
// registers); each wave keeps, for its rows, the
// running maximum m, the running sum l and the partial output in registers:
// the online softmax of the hotdry blog's section "3. 在线softmax算法"
// (initialise m = -inf and l = 0; for every key block raise the maximum,
// rescale the running sum and the partial output when it grew, add the
// block's exponentials and their weighted values).  Only O and
// lse = scale * m + ln l leave the chip (section "1. 内核融合策略": write only
// the final output; section "4. 重计算" keeps one statistic per row).
//
// Orientation: every product is computed transposed, S^T = K Q^T and
// O^T = V^T P^T, on the 32x32x16 MFMA, so that accumulator lane l belongs to
// query row l % 32: the row maximum, the row sum and the rescale factor are
// per-lane scalars, and the only cross-lane step is one exchange between
// lanes l and l ^ 32.  The exponentials leave the S^T accumulator directly as
// the B operand of the P.V product, and V^T is read from the V tile with the
// LDS transpose read.
//
// Software pipeline (per wave): while the matrix cores compute the scores of
// key tile j+1, the vector unit turns the scores of tile j into P (exp,
// running sum, packing); then the P.V products of tile j run.  Independent
// MFMA and VALU work of one wave overlap on the SIMD.
//
// Two running sums per row: l adds the fp32 exponentials and gives
// lse = scale * m + ln l; lh adds the same exponentials after their rounding
// to the 16-bit input type, i.e. exactly the weights the P.V product uses, and
// normalises O = (sum_j P_j V_j) / lh.  The weights of O then sum to one
// whatever the rounding of P: a row dominated by one key returns that key's
// value row instead of it scaled by the rounding error of its weight (up to
// 2^-9 relative in bf16, which for |V| > 5 alone exceeds a 1e-2 budget).
//
// Rescaling: the maximum m used for the exponentials is raised only when a
// row's new maximum exceeds it by more than 2^8 in the exponent (exp2 units);
// otherwise exponentials up to 2^8 are accumulated against the old m.  The
// online-softmax identity holds for any m the row uses consistently, so the
// result is the same up to rounding, and most tiles skip the rescale.
//
// Causal and window masking (snabindia chapter 1: the causal call skips the
// upper triangle): key tiles no row of the group sees are never loaded; only
// tiles at the edge of the visible band are masked element by element.  With
// a block mask (the same page's skipping of all-zero blocks, chapter 1 and
// section 3.1) the group visits only the key tiles of its active blocks.

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBK = 64;        // key rows per tile
// Query blocks (of 32 rows) per wave.  One block per wave with two waves per
// SIMD measured fastest: two blocks per wave halve the LDS reads per MFMA but
// need the output accumulators in AGPRs at one wave per SIMD, where the
// compiler also places the score accumulators and copies them back for the
// vector unit.
#ifndef ATTN_FWD_QB
#define ATTN_FWD_QB 1
#endif
constexpr float kLazy = 8.0f;  // rescale only when the maximum grows by more than 2^8

// Runs of unmasked key tiles at d = 128 go through a hand-scheduled loop
// (attn_fwd_loop.inc, written by gen_fwd_loop.py): the same instructions and
// accumulation order as the step below, so bitwise-equal results, with the
// vector work spread evenly between the MFMAs and the maximum of the next
// tile formed under this tile's P.V products.  ATTN_FWD_ASM=0 builds the
// kernel with the C++ step only.
#ifndef ATTN_FWD_ASM
#define ATTN_FWD_ASM 1
#endif
#if ATTN_FWD_ASM
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#include "attn_fwd_loop.inc"
#pragma clang diagnostic pop
#endif

// Maximum of 32 values as a tree of three-input maxima (depth 4 instead of a
// 31-long dependent chain).
__device__ inline float max32(const f32x16& a, const f32x16& b) {
    float t[11];
#pragma unroll
    for (int i = 0; i < 5; ++i) t[i] = fmaxf(fmaxf(a[3 * i], a[3 * i + 1]), a[3 * i + 2]);
#pragma unroll
    for (int i = 0; i < 5; ++i) t[5 + i] = fmaxf(fmaxf(b[3 * i], b[3 * i + 1]), b[3 * i + 2]);
    t[10] = fmaxf(a[15], b[15]);
    const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
    const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(t[9], t[10]);
    return fmaxf(fmaxf(u0, u1), fmaxf(u2, u3));
}

// KSPLIT = 2 (small grids): two sets of four waves share the group's query
// rows; set h walks the key tiles first + h, first + h + 2, ... with its own
// K/V buffers, and the two partial results merge at the end by the
// online-softmax rule (O = a0 O0 + a1 O1, l = a0 l0 + a1 l1, a_i = 2^(c (m_i - m))).
template <class T, int D, int QB, bool BS, int KSPLIT = 1>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads * KSPLIT, kThreads * KSPLIT),
                          amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
void attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, SeqLayout L, int ntq, float scale, float c, uint32_t qflip) {
    using DT = DmaTile<D, kBK>;
    constexpr int KS = D / 16;                 // MFMA k-steps of S^T over d
    constexpr int DB = D / 32;                 // 32-row blocks of O^T
    constexpr int TB = DT::BYTES / 2;          // tile size in 16-bit elements
    constexpr int STR = LdsStride<D>::value;   // row stride of the output staging
    constexpr int CH = D / 8;
    constexpr int BQ = kWaves * 32 * QB;       // query rows per work group
    constexpr int NT = kThreads * KSPLIT;
    static_assert(KSPLIT == 1 || (KSPLIT == 2 && QB == 1 && !BS), "key split: dense calls, one block per wave");
    constexpr int SMEM = (BQ * STR > 4 * TB * KSPLIT) ? BQ * STR : 4 * TB * KSPLIT;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = KSPLIT == 2 ? wave >> 2 : 0;  // key set of this wave
    const int w = KSPLIT == 2 ? wave & 3 : wave;   // its 32-row block
    const int n32 = lane & 31, h = lane >> 5;
    uint16_t* const Kb = smem + half * 4 * TB;  // K tiles: buffers 0, 1
    uint16_t* const Vb = Kb + 2 * TB;           // V tiles: buffers 0, 1

    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const Seq sq = resolve(L, item / ntq);
    const int qt = (L.wr >= 0 && L.wl < 0) ? ntq - 1 - item % ntq : item % ntq;
    const int q0 = qt * BQ;
    if (q0 >= sq.nq) return;  // the whole group: no barrier has been reached
    const int nq = sq.nq, nk = sq.nk;
    const uint16_t* Qh = Q + sq.qrow0 * D;
    const uint16_t* Kh = K + sq.krow0 * D;
    const uint16_t* Vh = V + sq.krow0 * D;
    const int wq0 = q0 + w * 32 * QB;  // block qb of this wave starts at row wq0 + 32 qb

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop;
    // qflip negates them (sign bits of both 16-bit halves) for a negative scale.
    u32x4 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = min(wq0 + 32 * qb + n32, nq - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = *(const u32x4*)(Qh + (int64_t)qrow * D + 16 * ks + 8 * h) ^ qflip;
    }

    const int qlast = min(q0 + BQ, nq) - 1;
    const TileRange tr = tile_range(sq.key_lo(q0), sq.key_hi(qlast), sq.key_lo(qlast),
                                    min(sq.key_hi(q0), nk - 1), nk, kBK);

    // Per-lane LDS read offsets (bytes, relative to a tile): K row fragments
    // (128-bit reads) and V^T operands (transpose reads).
    const uint32_t kofs[2] = {DT::frag_lane(lane, 0), DT::frag_lane(lane, 1)};
    const uint32_t vofs0 = DT::tr_lane(lane, 0), vofs1 = DT::tr_lane(lane, 1);
    const uint32_t goff = DT::lane_goff(lane);

    f32x16 oacc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[qb][db][e] = 0.f;
    // running maximum (raw score); this lane's shares of the running sums of
    // the exponentials (l) and of their 16-bit roundings (lh)
    float m[QB], l[QB], lh[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = kNegInf;
        l[qb] = 0.f;
        lh[qb] = 0.f;
    }
    f32x16 sacc[2][QB][2];  // scores of the tiles with even / odd index: [parity][query block][key block]

    // S^T(jt) = K(jt) Q^T into sacc[PAR], K(jt) in K buffer PAR.  Each K
    // fragment read from LDS feeds QB MFMAs.
    auto scores = [&](auto par_tag) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;
        const char* kt = (const char*)(Kb + PAR * TB);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[PAR][qb][kb][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = *(const u32x4*)(kt + kofs[ks & 1] + DT::frag_blk(kb, ks));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[PAR][qb][kb] = mfma32<T>(a, qf[qb][ks], sacc[PAR][qb][kb]);
            }
    };

    // With a block mask, only the key tiles of active (query block, key block)
    // pairs are visited, in order; the buffer parity then follows the position
    // in that walk instead of the tile index.  The mask is read with uniform
    // (scalar) loads.  A tile of 64 keys lies in mask block t / 2.
    static_assert(!BS || (BQ == kMaskBlock && 2 * kBK == kMaskBlock), "block masks need 128-row groups");
    const uint8_t* bmrow = BS ? sq.bm + (size_t)(q0 / kMaskBlock) * sq.nb : nullptr;
    auto next_tile = [&](int t) __attribute__((always_inline)) {
        ++t;
        if (BS)
            while (t < tr.end && !bmrow[t >> 1]) ++t;
        return t;
    };
    int j0 = tr.first + half;
    if (BS)
        while (j0 < tr.end && !bmrow[j0 >> 1]) ++j0;
    const int j1 = j0 < tr.end ? (KSPLIT == 2 ? min(j0 + 2, tr.end) : next_tile(j0)) : tr.end;
    // Buffer parity is the tile index parity.  With a block mask the visited
    // tiles still alternate in parity: an active block is the tile pair
    // (2b, 2b+1), so the walk only ever jumps from an odd tile to an even one
    // (clipping to [tr.first, tr.end) removes tiles only at its two ends).
    // With the key split, the buffer parity is the position in the set's walk.
    const int p0 = KSPLIT == 2 ? 0 : j0 & 1;

    // Prologue: tiles j0 (K, V) and j1 (K) in flight, then the scores of j0.
    if (j0 < tr.end) {
        dma_tile<D, kBK>(Kh, j0 * kBK, nk, Kb + p0 * TB, w, lane, goff);
        dma_tile<D, kBK>(Vh, j0 * kBK, nk, Vb + p0 * TB, w, lane, goff);
        if (j1 < tr.end) dma_tile<D, kBK>(Kh, j1 * kBK, nk, Kb + (1 - p0) * TB, w, lane, goff);
    }
    // Unconditional: the Q fragments and the first tiles have landed.  The
    // compiler counts only its own loads in vmcnt; waiting for everything
    // here keeps it from placing partial waits on the Q fragments inside the
    // loop, where the hardware counter also holds the prefetch DMA.
    wait_dma();
    __syncthreads();
    if (j0 < tr.end) {
        if (p0) scores(Flag<1>{});
        else scores(Flag<0>{});
    }

    // One key tile jt (buffer parity PAR): its scores are in sacc[PAR]; K(jn)
    // and V(jt) are in LDS, where jn and jn2 are the next two tiles visited.
    // MASKED: the tile crosses the edge of some row's visible band.  NEXT: a
    // tile jn exists.
    auto step = [&](int jt, int jn, int jn2, auto par_tag, auto masked_tag, auto next_tag)
                    __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;
        constexpr bool MASKED = decltype(masked_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
        const int k0 = jt * kBK;
        // Every wave has finished the previous tile (its K(jt) and V buffers
        // are free) and the DMA of K(jn), V(jt) has landed.
        __syncthreads();
        if (NEXT) {
            if (jn2 < tr.end) dma_tile<D, kBK>(Kh, jn2 * kBK, nk, Kb + PAR * TB, w, lane, goff);
            dma_tile<D, kBK>(Vh, jn * kBK, nk, Vb + (1 - PAR) * TB, w, lane, goff);
        }
        float mc[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            f32x16(&s)[2] = sacc[PAR][qb];
            if constexpr (MASKED) {
                const int qrow = wq0 + 32 * qb + n32;
                const int klo = sq.key_lo(qrow), khi = min(sq.key_hi(qrow), nk - 1);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key < klo || key > khi) s[kb][e] = kNegInf;
                    }
            }
            float mx = max32(s[0], s[1]);
            mx = max_with_other_half(mx);
            // Raise m (and rescale) only when the maximum grew by more than 2^8.
            const bool grow = mx > m[qb] && (m[qb] == kNegInf || (mx - m[qb]) * c > kLazy);
            if (__any(grow)) {
                const float mnew = fmaxf(m[qb], mx);
                const float alpha = (m[qb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m[qb] - mnew) * c);
                l[qb] *= alpha;
                lh[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
                m[qb] = mnew;
            }
            mc[qb] = (m[qb] == kNegInf) ? 0.f : m[qb] * c;
        }
        // Scores of the next tile on the matrix cores while P of this tile
        // is formed on the vector unit.  The wave issues this MFMA-heavy part
        // at raised priority, so that the other wave on the SIMD (in its
        // maximum and rescale code, or at the barrier) fills the gaps rather
        // than competing for issue slots (measured: 4-5% faster at d = 128).
        prio_mfma();
        if (NEXT) scores(Flag<1 - PAR>{});
        u32x4 pf[QB][2][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const f32x16& sv = sacc[PAR][qb][kb];
                f32x16 p;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], c, -mc[qb]));
                    if constexpr (MASKED) pe = sv[e] == kNegInf ? 0.f : pe;
                    p[e] = pe;
                }
                // the running sum adds the fp32 exponentials (four short chains)
                float l4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) l4[i] = (p[i] + p[i + 4]) + (p[i + 8] + p[i + 12]);
                l[qb] += (l4[0] + l4[1]) + (l4[2] + l4[3]);
                pack_acc_as_b<T>(p, pf[qb][kb][0], pf[qb][kb][1]);
                // the rounded weights, two per dword, in two chains
                float h0 = lh[qb], h1 = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h0 = add_pair<T>(pf[qb][kb][0][i], h0);
                    h1 = add_pair<T>(pf[qb][kb][1][i], h1);
                }
                lh[qb] = h0 + h1;
            }
        // O^T += V^T P^T: each V^T fragment read from LDS feeds QB MFMAs
        const char* vt = (const char*)(Vb + PAR * TB);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 a = tr_operand_dma(vt, vofs0, vofs1, DT::tr_blk(2 * kb + t, db));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32<T>(a, pf[qb][kb][t], oacc[qb][db]);
                }
        prio_normal();
        wait_dma();
    };

    if constexpr (KSPLIT == 2) {
        // Position k of set `half` is tile first + half + 2k, in buffers k & 1.
        // Both sets run n0 steps (one barrier each); a set with one tile
        // fewer ends on a bare barrier.
        const int nt = tr.end - tr.first;
        const int n0 = (nt + 1) >> 1, nh = (nt + 1 - half) >> 1;
        auto tile_at = [&](int k) __attribute__((always_inline)) { return tr.first + half + 2 * k; };
        // number of positions whose tile lies below t
        auto pos_of = [&](int t) __attribute__((always_inline)) { return max(0, (t - tr.first - half + 1) >> 1); };
        if (nh > 0) {
            const int lastk = nh - 1;
            // positions [ka, kb) of one kind, each with a successor
            auto run = [&](int ka, int kb, auto masked_tag) __attribute__((always_inline)) {
                int k = ka;
                if (k < kb && (k & 1)) {
                    step(tile_at(k), tile_at(k + 1), tile_at(k + 2), Flag<1>{}, masked_tag, Flag<true>{});
                    ++k;
                }
                for (; k + 1 < kb; k += 2) {
                    step(tile_at(k), tile_at(k + 1), tile_at(k + 2), Flag<0>{}, masked_tag, Flag<true>{});
                    step(tile_at(k + 1), tile_at(k + 2), tile_at(k + 3), Flag<1>{}, masked_tag, Flag<true>{});
                }
                if (k < kb) step(tile_at(k), tile_at(k + 1), tile_at(k + 2), Flag<0>{}, masked_tag, Flag<true>{});
            };
            const int kff = min(pos_of(tr.full_first), lastk);
            const int kfe = min(max(pos_of(tr.full_end), kff), lastk);
            run(0, kff, Flag<true>{});
            run(kff, kfe, Flag<false>{});
            run(kfe, lastk, Flag<true>{});
            const int last = tile_at(lastk);
            const bool last_masked = last < tr.full_first || last >= tr.full_end;
            if (lastk & 1) {
                if (last_masked) step(last, tr.end, tr.end, Flag<1>{}, Flag<true>{}, Flag<false>{});
                else step(last, tr.end, tr.end, Flag<1>{}, Flag<false>{}, Flag<false>{});
            } else {
                if (last_masked) step(last, tr.end, tr.end, Flag<0>{}, Flag<true>{}, Flag<false>{});
                else step(last, tr.end, tr.end, Flag<0>{}, Flag<false>{}, Flag<false>{});
            }
        }
        if (nh < n0) __syncthreads();
    } else if constexpr (!BS) {
        // Tiles [a, b) all of one kind (masked or not), none of them the last.
        auto run = [&](int a, int b, auto masked_tag) __attribute__((always_inline)) {
            int jt = a;
            if (jt < b && (jt & 1)) {
                step(jt, jt + 1, jt + 2, Flag<1>{}, masked_tag, Flag<true>{});
                ++jt;
            }
            for (; jt + 1 < b; jt += 2) {
                step(jt, jt + 1, jt + 2, Flag<0>{}, masked_tag, Flag<true>{});
                step(jt + 1, jt + 2, jt + 3, Flag<1>{}, masked_tag, Flag<true>{});
            }
            if (jt < b) step(jt, jt + 1, jt + 2, Flag<0>{}, masked_tag, Flag<true>{});
        };
        if (tr.end > tr.first) {
            const int last = tr.end - 1;
            run(tr.first, min(tr.full_first, last), Flag<true>{});
            int ua = tr.full_first;
            const int ub = min(tr.full_end, last);
#if ATTN_FWD_ASM
            if constexpr (QB == 1 && D == 128) {
                // Tiles [ua, bb) through the hand-scheduled loop: unmasked, each with
                // a successor, and K(jt + 2), V(jt + 1) whole tiles (its DMA has no
                // clamped rows).  The loop enters with S(ua) computed and K(ua + 1),
                // V(ua) in flight, and leaves the state the step below expects.
                const int bb = min(ub, min(tr.end, nk / kBK) - 2);
                if (bb > ua) {
                    const uint32_t sl = lds_addr(Kb);
                    const uint32_t mk0 = __builtin_amdgcn_readfirstlane(sl + w * 1024);
                    const uint32_t mv0 = mk0 + 2 * DT::BYTES;
                    const int rg = w / DT::CG, cg = w % DT::CG;
                    const uint64_t wofs = (uint64_t)((rg * 16 * D + cg * 32) * 2);
                    const uint64_t kb64 = (uint64_t)(uintptr_t)Kh + (uint64_t)(ua + 2) * DT::BYTES + wofs;
                    const uint64_t vb64 = (uint64_t)(uintptr_t)Vh + (uint64_t)(ua + 1) * DT::BYTES + wofs;
                    // readfirstlane returns a signed int: each half goes through uint32_t,
                    // or a low word with bit 31 set would sign-extend into the high word
                    const uint64_t kbs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)kb64) |
                                         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(kb64 >> 32)) << 32);
                    const uint64_t vbs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)vb64) |
                                         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(vb64 >> 32)) << 32);
                    const uint32_t g[4] = {goff, goff + 4096, goff + 8192, goff + 12288};
                    fwd_unmasked_run<T, D>(oacc[0], sacc[0][0], sacc[1][0], m[0], l[0], lh[0], qf[0], sl + kofs[0],
                                           sl + kofs[1], sl + vofs0, sl + vofs1, g, c, (uint32_t)(ua & 1), mk0,
                                           mk0 + DT::BYTES, mv0, mv0 + DT::BYTES, kbs, vbs, (uint32_t)(bb - ua));
                    ua = bb;
                }
            }
#endif
            run(ua, ub, Flag<false>{});
            run(max(tr.full_end, tr.full_first), last, Flag<true>{});
            const bool last_masked = last < tr.full_first || last >= tr.full_end;
            if (last & 1) {
                if (last_masked) step(last, tr.end, tr.end, Flag<1>{}, Flag<true>{}, Flag<false>{});
                else step(last, tr.end, tr.end, Flag<1>{}, Flag<false>{}, Flag<false>{});
            } else {
                if (last_masked) step(last, tr.end, tr.end, Flag<0>{}, Flag<true>{}, Flag<false>{});
                else step(last, tr.end, tr.end, Flag<0>{}, Flag<false>{}, Flag<false>{});
            }
        }
    } else {
        // Walk the active tiles: two steps per iteration, of fixed parities,
        // as in the dense loop, and the last tile (which has no successor)
        // after the loops.  Masked tiles (those some row of the group does
        // not see whole) lie before full_first or from full_end on; the
        // interior tiles of active blocks take the unmasked step.  One loop
        // per kind: a loop whose body branched between the two kinds would
        // have the compiler copy the accumulators every tile.
        int jt = j0, jn = j1;
        // Steps for the tiles jt < lim that have a successor.
        auto run = [&](int lim, auto masked_tag) __attribute__((always_inline)) {
            if (jt < lim && jn < tr.end && (jt & 1)) {
                const int jn2 = next_tile(jn);
                step(jt, jn, jn2, Flag<1>{}, masked_tag, Flag<true>{});
                jt = jn;
                jn = jn2;
            }
            while (jt < lim && jn < tr.end) {  // jt is even
                int jn2 = next_tile(jn);
                step(jt, jn, jn2, Flag<0>{}, masked_tag, Flag<true>{});
                jt = jn;
                jn = jn2;
                if (jt >= lim || jn >= tr.end) break;
                jn2 = next_tile(jn);
                step(jt, jn, jn2, Flag<1>{}, masked_tag, Flag<true>{});
                jt = jn;
                jn = jn2;
            }
        };
        run(tr.full_first, Flag<true>{});
        run(tr.full_end, Flag<false>{});
        run(tr.end, Flag<true>{});
        if (jt < tr.end) {  // the last tile
            const bool last_masked = jt < tr.full_first || jt >= tr.full_end;
            if (jt & 1) {
                if (last_masked) step(jt, tr.end, tr.end, Flag<1>{}, Flag<true>{}, Flag<false>{});
                else step(jt, tr.end, tr.end, Flag<1>{}, Flag<false>{}, Flag<false>{});
            } else {
                if (last_masked) step(jt, tr.end, tr.end, Flag<0>{}, Flag<true>{}, Flag<false>{});
                else step(jt, tr.end, tr.end, Flag<0>{}, Flag<false>{}, Flag<false>{});
            }
        }
    }
    __syncthreads();  // every wave is done with the tile buffers

    if constexpr (KSPLIT == 2) {
        // merge the second set's partial result into the first set's
        float* xo = (float*)smem;            // [row block][DB][16][lane]: O^T of set 1
        float* xs = xo + 4 * DB * 16 * 64;   // [row block][m, l, lh][lane]
        if (half == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) xo[((w * DB + db) * 16 + e) * 64 + lane] = oacc[0][db][e];
            xs[(w * 3 + 0) * 64 + lane] = m[0];
            xs[(w * 3 + 1) * 64 + lane] = l[0];
            xs[(w * 3 + 2) * 64 + lane] = lh[0];
        }
        __syncthreads();
        if (half == 0) {
            const float m1 = xs[(w * 3 + 0) * 64 + lane];
            const float l1 = xs[(w * 3 + 1) * 64 + lane];
            const float lh1 = xs[(w * 3 + 2) * 64 + lane];
            const float mm = fmaxf(m[0], m1);
            const float a0 = m[0] == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m[0] - mm) * c);
            const float a1 = m1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * c);
            l[0] = a0 * l[0] + a1 * l1;
            lh[0] = a0 * lh[0] + a1 * lh1;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[0][db][e] = a0 * oacc[0][db][e] + a1 * xo[((w * DB + db) * 16 + e) * 64 + lane];
            m[0] = mm;
        }
        __syncthreads();  // the merge area is the staging area below
    }

    // ---- epilogue: O = O^T / l, staged through LDS for row-contiguous stores
    uint16_t* Os = smem;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if (half != 0) break;
        const int qrow = wq0 + 32 * qb + n32;
        const float lt = sum_with_other_half(l[qb]);
        const float lht = sum_with_other_half(lh[qb]);
        // a row that sees no key at all: O = 0, lse = -inf
        const float inv = lht > 0.f ? 1.f / lht : 0.f;
        if (h == 0 && qrow < nq) LSE[sq.qrow0 + qrow] = lt > 0.f ? m[qb] * scale + logf(lt) : kNegInf;
        const int orow = (w * 32 * QB + 32 * qb + n32) * STR;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 pk = {pack2<T>(oacc[qb][db][4 * g] * inv, oacc[qb][db][4 * g + 1] * inv),
                            pack2<T>(oacc[qb][db][4 * g + 2] * inv, oacc[qb][db][4 * g + 3] * inv)};
                *(u32x2*)(Os + orow + 32 * db + 8 * g + 4 * h) = pk;
            }
    }
    __syncthreads();
    uint16_t* Oh = O + sq.qrow0 * D;
    for (int ch = tid; ch < BQ * CH; ch += NT) {
        const int r = ch / CH, col = ch % CH;
        if (q0 + r < nq) *(u32x4*)(Oh + (int64_t)(q0 + r) * D + 8 * col) = *(const u32x4*)(Os + r * STR + 8 * col);
    }
}

// Compute units of the device a stream belongs to (cached per device).
int cu_count(void* stream) {
    static int cache[64];
    int dev = 0;
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v <= 0) {
        int n = 0;
        v = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
        __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}

template <class T, int D, bool BS>
hipError_t launch(const FwdParams& p) {
    constexpr int QB = BS ? 1 : ATTN_FWD_QB, BQ = kWaves * 32 * QB;
    // A negative scale runs as |scale| with Q negated (a sign flip, exact in
    // 16-bit storage): scale * <q, k> = |scale| * <-q, k> bit for bit, so the
    // running maximum is always taken of the logits that the exponentials use.
    const bool neg = p.scale < 0.f;
    const float ascale = neg ? -p.scale : p.scale;
    const uint32_t qflip = neg ? 0x80008000u : 0u;
    const int ntq = (p.max_nq + BQ - 1) / BQ;
    const int64_t nseq = (int64_t)p.L.B * p.L.H;
    const int64_t blocks = nseq * ntq;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // A grid that gives each CU at most one group of four waves leaves every
    // SIMD with a single wave: split each group's keys over two wave sets
    // instead (eight waves per group, half the walk per set).
    if (!BS && QB == 1 && blocks <= cu_count(p.stream)) {
        hipLaunchKernelGGL((attn_fwd_kernel<T, D, 1, false, 2>), dim3((unsigned)blocks), dim3(2 * kThreads), 0,
                           (hipStream_t)p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                           (const uint16_t*)p.v, (uint16_t*)p.o, p.lse, p.L, ntq, ascale, ascale * kLog2e, qflip);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, QB, BS>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                       (const uint16_t*)p.v, (uint16_t*)p.o, p.lse, p.L, ntq, ascale,
                       ascale * kLog2e, qflip);
    return hipGetLastError();
}

template <class T, bool BS>
hipError_t launch_d(const FwdParams& p) {
    return p.d == 64 ? launch<T, 64, BS>(p) : launch<T, 128, BS>(p);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p) {
    if (p.L.bmask) return p.dtype == kDtypeBF16 ? launch_d<BF16, true>(p) : launch_d<F16, true>(p);
    return p.dtype == kDtypeBF16 ? launch_d<BF16, false>(p) : launch_d<F16, false>(p);
}

}  // namespace attn
