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

// ---------------------------------------------------------------------------
// Tiles loaded by DMA (global_load_lds_dwordx4: global memory straight into
// LDS, no registers).
//
// LDS image of a ROWS x D tile of 16-bit values: the tile is cut into blocks
// of 16 rows x 4 chunks (a chunk is 8 values, 16 bytes); block (rg, cg) sits at
// byte (rg * CG + cg) * 1024, CG = D / 32.  Inside a block, row r takes 64
// bytes at r * 64 and its chunk c is stored in slot c ^ ((r >> 2) & 3).  One
// wave-wide DMA instruction fills one block (lane L writes bytes 16 L ..
// 16 L + 15, i.e. row L / 4, slot L % 4), so every global read is 16 rows x 64
// contiguous bytes.  The slot swizzle makes both LDS read patterns of the
// kernels conflict-free: 16 lanes reading one chunk of 16 consecutive rows
// (128-bit reads of MFMA row fragments) and 16 lanes reading 4 rows x 32 bytes
// (transpose reads) each touch 16 distinct bank groups.
template <int D, int ROWS>
struct DmaTile {
    static constexpr int CG = D / 32;                 // chunk groups per row
    static constexpr int BYTES = ROWS * D * 2;        // one tile
    static constexpr int ELEMS = ROWS * D;
    static constexpr int NBLK = (ROWS / 16) * CG;     // 1 KB blocks per tile
    static constexpr int PER_WAVE = NBLK / 4;         // DMA instructions per wave (4 waves)
    static_assert(NBLK % 4 == 0, "tile blocks must split over four waves");

    // Byte offset, inside the global tile, of the chunk this lane loads for
    // a block (excluding the block's base).
    __device__ static inline uint32_t lane_goff(int lane) {
        const int r = lane >> 2, c = (lane & 3) ^ ((r >> 2) & 3);
        return (uint32_t)(r * D + c * 8) * 2u;
    }

    // 128-bit read of an MFMA row fragment: row 32 rb + n32 (n32 = lane % 32),
    // chunk 2 ks + lane / 32.  frag_lane(lane, ks & 1) + frag_blk(rb, ks)
    // (bytes; the lane part is loop-invariant, the block part a constant).
    __device__ static inline uint32_t frag_lane(int lane, int p) {
        const int n32 = lane & 31, h = lane >> 5, r = n32 & 15;
        return (uint32_t)((n32 >> 4) * CG * 1024 + r * 64 + (((2 * p + h) ^ ((r >> 2) & 3)) << 4));
    }
    static constexpr int frag_blk(int rb, int ks) { return (2 * rb * CG + ks / 2) * 1024; }

    // Transpose read e (e = 0, 1) yielding half of the A operand
    // A[m][k] = T[16 rs + k][32 db + m] of a 32x32x16 MFMA (see lds_read_tr):
    // tr_lane(lane, e) + tr_blk(rs, db).
    __device__ static inline uint32_t tr_lane(int lane, int e) {
        const int h = lane >> 5, g16 = lane & 15, x = (lane >> 4) & 1;
        const int row = 8 * e + 4 * h + (g16 >> 2);
        const int cc = 2 * x + ((g16 & 3) >> 1);
        return (uint32_t)(row * 64 + ((cc ^ (2 * e + h)) << 4) + (g16 & 1) * 8);
    }
    static constexpr int tr_blk(int rs, int db) { return (rs * CG + db) * 1024; }
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One DMA instruction: 16 bytes per lane from base + voff (global) into LDS at
// lds_byte + 16 * lane.  Issued in assembly: the compiler does not track it,
// so it neither waits for it before unrelated LDS reads nor reuses LDS values
// across it ("memory" clobber); kernels wait with wait_dma() and a barrier
// before any wave reads the tile.  M0 carries the LDS address and needs one
// wait state after being written.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(const void* base, uint32_t voff, uint32_t lds_byte) {
    // base and lds_byte are wave-uniform; make that explicit for the SGPR operands
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
    const void* sbase = (const void*)(uintptr_t)sb;
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(lds_byte);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt(0): every DMA (and global load) of this wave has landed; expcnt and
// lgkmcnt are not waited on.
__device__ inline void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Issue the DMA of rows r0 .. r0+ROWS-1 of a [nrows, D] array into an LDS
// tile (four waves share the work; w is the wave-uniform wave index).  Rows
// at or beyond nrows read row nrows-1 (callers mask or discard them).
template <int D, int ROWS>
__device__ inline void dma_tile(const uint16_t* __restrict__ src, int r0, int nrows, const uint16_t* lds_tile,
                                int w, int lane, uint32_t goff) {
    using DT = DmaTile<D, ROWS>;
    const char* base = (const char*)(src + (int64_t)r0 * D);
    const uint32_t lt = lds_addr(lds_tile);
    if (r0 + ROWS <= nrows) {
#pragma unroll
        for (int i = 0; i < DT::PER_WAVE; ++i) {
            const int b = w + 4 * i, rg = b / DT::CG, cg = b % DT::CG;
            dma16(base + (rg * 16 * D + cg * 32) * 2, goff, lt + b * 1024);
        }
    } else {
        const int r = lane >> 2, c = (lane & 3) ^ ((r >> 2) & 3);
#pragma unroll
        for (int i = 0; i < DT::PER_WAVE; ++i) {
            const int b = w + 4 * i, rg = b / DT::CG, cg = b % DT::CG;
            const int row = min(rg * 16 + r, nrows - 1 - r0);
            dma16(base, (uint32_t)(row * D + cg * 32 + c * 8) * 2u, lt + b * 1024);
        }
    }
}

// A operand of a 32x32x16 MFMA read transposed from a DMA tile (two transpose
// reads; tile_at is the tile's byte address, ofs0/ofs1 the tr_lane offsets).
__device__ inline u32x4 tr_operand_dma(const char* tile, uint32_t ofs0, uint32_t ofs1, int blk) {
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + ofs0 + blk)));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + ofs1 + blk)));
    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
    return a;
}

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

// a.lo + a.hi + acc for a dword holding two 16-bit values (v_dot2c against
// (1, 1); the products are exact, the sum is taken in fp32).
template <class T>
__device__ inline float add_pair(uint32_t a, float acc);

template <>
__device__ inline float add_pair<BF16>(uint32_t a, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
}

template <>
__device__ inline float add_pair<F16>(uint32_t a, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
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
    const uint8_t* bm;  // block mask of this sequence, [nb, nb] (nullptr: none)
    int nb;

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
    r.bm = nullptr;
    r.nb = L.bm_nb;
    if (L.mode == 0) {
        r.qrow0 = r.krow0 = (int64_t)s * L.N;
        r.nq = r.nk = L.N;
        r.off = 0;
        if (L.bmask) {
            const int m = L.bm_heads == 1 ? 0 : (L.bm_heads == L.H ? s % L.H : s);
            r.bm = L.bmask + (size_t)m * L.bm_nb * L.bm_nb;
        }
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
