// attn_device.h -- gfx950 building blocks shared by the attention kernels:
// vector types, the 16-bit MFMA in its two input types, round-to-nearest-even
// packing of fp32 pairs, LDS transpose reads, the cross-half lane exchange
// and the XCD-aware work-group remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
