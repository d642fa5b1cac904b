// attn_device.h -- gfx950 building blocks shared by the attention kernels:
// vector types, the 16-bit MFMA in its two input types, round-to-nearest-even
// packing of fp32 pairs, LDS transpose reads, the cross-half lane exchange
// and the XCD-aware work-group remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Element-type tags: the storage of Q/K/V/O is 16-bit either way.
struct BF16 {};
struct F16 {};

constexpr float kLog2e = 1.4426950408889634f;

// Compile-time flag passed to generic lambdas (e.g. masked / unmasked tiles).
template <bool B>
struct Flag {
    static constexpr bool value = B;
};
constexpr float kNegInf = -__builtin_inff();

// D(32x32, fp32) += A(32x16) * B(16x32), 16-bit inputs.
// Lane l holds A[l%32][8*(l/32) .. +7], B[8*(l/32) .. +7][l%32] and
// D[8*(e/4) + 4*(l/32) + e%4][l%32] for e = 0..15.
template <class T>
__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ inline f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ inline f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> two 16-bit values in one dword (lo in bits 0..15),
// round to nearest even.
template <class T>
__device__ inline uint32_t pack2(float lo, float hi);

template <>
__device__ inline uint32_t pack2<BF16>(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <>
__device__ inline uint32_t pack2<F16>(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j supplies the address of four consecutive 16-bit values; lane i then
// receives, as its element k (k = 0..3), value i%4 of the four supplied by
// lane 4k + i/4.  When lane j = 4k + r points at row (base + k), columns
// (c0 + 4r .. c0 + 4r + 3) of a row-major array, lane i receives column
// c0 + i of rows base .. base + 3: a 4 x 16 block read transposed.
__device__ inline u32x2 lds_read_tr(const uint16_t* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Exchange between the two 32-lane halves of a wave (v_permlane32_swap):
// lanes 32..63 of `a` trade places with lanes 0..31 of `b`.  Called with
// a == b == x, every lane ends up holding {x[l], x[l ^ 32]} in {a, b}, so
// max(a, b) and a + b combine a row's two halves symmetrically.
// Written as inline assembly: this compiler folds the two results of
// __builtin_amdgcn_permlane32_swap into one when both feed the same
// arithmetic instruction.  The s_nop 1 on either side gives the two wait
// states the compiler itself places before the swap.
__device__ inline void swap_halves(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

__device__ inline float max_with_other_half(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    swap_halves(a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ inline float sum_with_other_half(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    swap_halves(a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// LDS row stride (in 16-bit elements) of a tile with D columns.  LDS has 64
// banks of 4 bytes; a 128-bit read is served 16 lanes at a time, and a
// transpose read serves 16-lane groups that each touch 4 rows x 32 bytes.
// A stride of 76 dwords (D = 128) or 36 dwords (D = 64) keeps both access
// kinds free of bank conflicts (measured on gfx950: ~200 B/clk/CU for
// 128-bit reads, ~100 B/clk/CU for transpose reads).
template <int D>
struct LdsStride;
#ifndef ATTN_LDS_STRIDE_128
#define ATTN_LDS_STRIDE_128 152
#endif
template <>
struct LdsStride<128> {
    static constexpr int value = ATTN_LDS_STRIDE_128;
};
template <>
struct LdsStride<64> {
    static constexpr int value = 72;
};

// Copy a tile of ROWS x D 16-bit values (rows r0 .. r0+ROWS-1 of a row-major
// [nrows, D] array, nrows >= 1) from global memory into registers, 16 bytes
// per chunk, then into an LDS tile of row stride LdsStride<D>.
//
// Each thread's chunk offsets inside a tile are computed once and stay in
// registers for the whole loop; the tile's base address is wave-uniform.  A
// load is then one instruction on an SGPR base plus a fixed VGPR offset, and
// no address register is ever recycled while a prefetch is still in flight
// (recycling one makes the compiler wait for that prefetch before the next
// use of the register).  Rows at or beyond nrows read row nrows-1 instead, so
// every load stays in bounds without exec-mask branches; callers mask or
// discard the duplicated rows.  THREADS threads split the tile.
template <int ROWS, int D, int THREADS>
struct TileCopy {
    static constexpr int CH = D / 8;                      // 16-byte chunks per row
    static constexpr int CPT = ROWS * CH / THREADS;       // chunks per thread
    static_assert(ROWS * CH % THREADS == 0, "tile must split evenly over the threads");
    static constexpr int STR = LdsStride<D>::value;

    u32x4 r[CPT];
    uint32_t goff[CPT];  // byte offset of chunk i inside a global tile
    uint32_t loff[CPT];  // element offset of chunk i inside an LDS tile

    __device__ inline explicit TileCopy(int tid) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * THREADS;
            goff[i] = (uint32_t)((c / CH) * D + 8 * (c % CH)) * 2u;
            loff[i] = (uint32_t)((c / CH) * STR + 8 * (c % CH));
        }
    }

    __device__ inline void load(const uint16_t* __restrict__ src, int r0, int nrows, int tid) {
        const char* base = (const char*)(src + (int64_t)r0 * D);
        if (r0 + ROWS <= nrows) {
#pragma unroll
            for (int i = 0; i < CPT; ++i) r[i] = *(const u32x4*)(base + goff[i]);
        } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = tid + i * THREADS;
                const int row = min(c / CH, nrows - 1 - r0);
                r[i] = *(const u32x4*)(base + (uint32_t)(row * D + 8 * (c % CH)) * 2u);
            }
        }
    }

    __device__ inline void store(uint16_t* dst) const {
#pragma unroll
        for (int i = 0; i < CPT; ++i) *(u32x4*)(dst + loff[i]) = r[i];
    }
};

// Offset (in elements, relative to the start of a 32-column block of a 16-row
// step) of this lane's address for the transpose read that yields the A
// operand A[m][k] = T[row(k)][col0 + m] of a 32x32x16 MFMA from a row-major
// LDS tile T: 16-lane group g reads columns 16*(g%2) .. +15 and rows
// 4*(lane/32) .. +3; a second read 8 rows further supplies k = 4..7.  With
// this, logical k = 8*(l/32) + e maps to row 8*(e/4) + 4*(l/32) + e%4 of the
// step, which is exactly the row order of a 32x32 accumulator's elements.
template <int STR>
__device__ inline int tr_lane_offset(int lane) {
    const int g16 = lane & 15;
    return ((g16 >> 2) + 4 * (lane >> 5)) * STR + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
}

// A operand (M = 32 columns starting at col0, K = 16 rows starting at row0)
// read transposed from a row-major LDS tile, for the lane offset above.
template <int STR>
__device__ inline u32x4 tr_operand(const uint16_t* tile_at_lane, int row0, int col0) {
    const uint16_t* p = tile_at_lane + row0 * STR + col0;
    const u32x2 lo = lds_read_tr(p);
    const u32x2 hi = lds_read_tr(p + 8 * STR);
    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
    return a;
}

// Pack the 16 fp32 accumulator values of a 32x32 MFMA result (lane l: column
// l % 32, rows 8*(e/4) + 4*(l/32) + e%4) into the B operands of two 16-deep
// k-steps that contract over those rows: k-step t takes elements 8t .. 8t+7.
template <class T>
__device__ inline void pack_acc_as_b(const f32x16& v, u32x4& b0, u32x4& b1) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        b0[e >> 1] = pack2<T>(v[e], v[e + 1]);
        b1[e >> 1] = pack2<T>(v[8 + e], v[8 + e + 1]);
    }
}

// Scheduling groups for a run of NMFMA MFMAs fed by LDS reads: the first
// AHEAD reads are issued up front, then each MFMA is followed by the next
// PER reads, so every MFMA finds its operands loaded AHEAD/PER MFMAs earlier.
template <int AHEAD, int NMFMA, int PER>
__device__ inline void sched_reads_ahead() {
    constexpr int later = NMFMA * PER - AHEAD;  // reads issued between MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < later / PER) __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
    }
}

// Issue priority around MFMA runs: the wave issuing MFMAs is preferred, so
// the other wave on the SIMD fills the gaps with VALU work.
__device__ inline void prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ inline void prio_normal() { __builtin_amdgcn_s_setprio(0); }

// One sequence of a call, resolved on the device (see SeqLayout).
struct Seq {
    int64_t qrow0, krow0;  // global row index of query row 0 / key row 0
    int nq, nk;
    int off;     // query row i sits at key position i + off
    int wl, wr;  // window bounds (-1: unbounded)

    // First and last key (inclusive, before clipping to [0, nk)) visible to row i.
    __device__ inline int key_lo(int i) const { return wl < 0 ? -0x3fffffff : i + off - wl; }
    __device__ inline int key_hi(int i) const { return wr < 0 ? 0x3fffffff : i + off + wr; }
    // First and last query row (inclusive, before clipping) that sees key j.
    __device__ inline int row_lo(int j) const { return wr < 0 ? -0x3fffffff : j - off - wr; }
    __device__ inline int row_hi(int j) const { return wl < 0 ? 0x3fffffff : j - off + wl; }
    __device__ inline bool visible(int i, int j) const {
        return j >= key_lo(i) && j <= key_hi(i);
    }
};

__device__ inline Seq resolve(const SeqLayout& L, int s) {
    Seq r;
    r.wl = L.wl;
    r.wr = L.wr;
    if (L.mode == 0) {
        r.qrow0 = r.krow0 = (int64_t)s * L.N;
        r.nq = r.nk = L.N;
        r.off = 0;
        return r;
    }
    const int h = s / L.B, b = s % L.B;
    const int q0 = min(max(L.cu_q[b], 0), L.total_q), q1 = min(max(L.cu_q[b + 1], q0), L.total_q);
    const int k0 = min(max(L.cu_k[b], 0), L.total_k), k1 = min(max(L.cu_k[b + 1], k0), L.total_k);
    r.qrow0 = (int64_t)h * L.total_q + q0;
    r.krow0 = (int64_t)h * L.total_k + k0;
    r.nq = q1 - q0;
    r.nk = k1 - k0;
    r.off = r.nk - r.nq;
    return r;
}

// Tiles [first, end) of size BT that hold an index in [lo, hi] (inclusive,
// clipped to [0, n); empty when nothing is left), and the sub-range
// [full_first, full_end) of those tiles whose every index lies in
// [all_lo, all_hi] (the caller clips all_hi as the use requires).
struct TileRange {
    int first, end, full_first, full_end;
};

__device__ inline TileRange tile_range(int lo, int hi, int all_lo, int all_hi, int n, int bt) {
    TileRange t;
    lo = max(lo, 0);
    hi = min(hi, n - 1);
    if (hi < lo) {
        t.first = t.end = t.full_first = t.full_end = 0;
        return t;
    }
    t.first = lo / bt;
    t.end = hi / bt + 1;
    all_lo = max(all_lo, 0);
    int ff = (all_lo + bt - 1) / bt, fe = all_hi < all_lo ? ff : (all_hi + 1) / bt;
    ff = min(max(ff, t.first), t.end);
    fe = min(max(fe, ff), t.end);
    t.full_first = ff;
    t.full_end = fe;
    return t;
}

// Work groups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber them so that each XCD receives one contiguous range of work items:
// consecutive items (the tiles of one head) then share that XCD's L2.
// A bijection on [0, n) for any n.
__device__ inline int xcd_contiguous(int b, int n) {
    const int q = n >> 3, r = n & 7;
    const int xcd = b & 7, local = b >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

}  // namespace attn
