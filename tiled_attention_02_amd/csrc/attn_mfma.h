// gfx950 matrix-core helpers shared by the forward and backward kernels: operand vector
// types, the 32x32x16 bf16/fp16 MFMA with its pack / dot helpers, the row permutation
// sigma that makes a product's accumulator registers the operand of the next product, and
// the K/V tile swizzles and global -> LDS copy of the forward kernels.
//
// v_mfma_f32_32x32x16_{bf16,f16} lane layouts (lane l, half h = l / 32):
//   A (32 x 16): lane l holds row l % 32, k = 8h .. 8h + 7 (one u32x4 of 8 elements)
//   B (16 x 32): lane l holds column l % 32, k = 8h .. 8h + 7
//   C (32 x 32): register r of lane l holds row 8 (r / 4) + 4h + r % 4, column l % 32
// Feeding A's rows in the order sigma(m) (bits 2 and 3 swapped) makes register r of half h
// hold row 16 (r / 8) + 8h + r % 8: registers 8kk .. 8kk + 7 are then exactly the k-slots
// 16kk + 8h .. + 7 of a B operand whose k index is that row index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"

namespace aule {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
    }
    // acc + lo + hi of a packed pair, in fp32 (v_dot2 against (1, 1))
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const bf16x2 one = {(bf16_t)1.0f, (bf16_t)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
    }
    // acc + a.lo * b.lo + a.hi * b.hi of two packed pairs, in fp32
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
    }
};
template <> struct Mfma<f16_t> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // two fp32 -> packed fp16 pair, round to nearest even (one v_cvt_pk_f16_f32)
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
    }
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const f16x2 one = {(f16_t)1.0f, (f16_t)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
    }
};

// sigma: swap bits 2 and 3 (an involution on 0..31)
__device__ __forceinline__ int sigma(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk swizzles (XOR on the chunk index inside a row) of K and V tiles in LDS.
// K rows: the S^T reads of one instruction hit rows sigma(0..31) at one column; chunk c of
//   row r sits at c ^ kswz(r) with kswz(r) = kx_lane(sigma(r % 32)), the mask of the lane
//   that reads row r (sigma is an involution). Each group of 16 lanes (one 256-byte pass of
//   the LDS banks) must hit 16 distinct 16-byte slots: with 16 chunks per row (256-byte rows)
//   kx_lane(l) = l % 16 does that; with 8 chunks (128-byte rows, two rows per bank row) the
//   row's parity (l % 2, which sigma keeps) picks the half and kx_lane(l) = (l / 2) % 8 the
//   chunk (l % 8 there left lanes l and l + 8 on one slot: 2-way conflicts).
// V rows: a transposed read touches 4 consecutive rows x 2 (or 4) neighbouring chunks; the
//   per-row XOR masks below make those slots distinct modulo 8 and modulo 16 chunks.
template <int KC> __device__ __forceinline__ int kx_lane(int l32) {
    static_assert(KC == 8 || KC == 16, "rows of 8 or 16 chunks");
    return KC == 16 ? (l32 & 15) : ((l32 >> 1) & 7);
}
template <int KC> __device__ __forceinline__ int kswz(int row) { return kx_lane<KC>(sigma(row & 31)); }
template <int KC> __device__ __forceinline__ int vswz(int row) {
    if constexpr (KC == 16) return (0xCA60 >> (4 * (row & 3))) & 15;   // 0, 6, 10, 12
    else return 2 * (row & 3);
}

[[maybe_unused]] constexpr uint32_t kBufferFlags = 0x00020000u;   // raw buffer, 32-bit data format
[[maybe_unused]] constexpr uint32_t kOobOffset = 0x7FFFFFF0u;     // an offset past any slice: reads as zero

#if defined(__HIP_DEVICE_COMPILE__)
// One 16-byte global -> LDS copy per lane: LDS[m0 + 16 * lane] = buffer[voffset], zero when
// voffset lies past the descriptor's size. Written as inline asm so the compiler does not
// track it: its alias analysis cannot tell the destination buffer from the buffers being
// read and would otherwise wait for every copy right after issuing it. Completion is
// ordered explicitly instead (s_waitcnt vmcnt, plus s_barrier when other waves read the
// data). M0 is saved and restored around the copy.
__device__ __forceinline__ void lds_copy16(i32x4 rsrc, uint32_t voffset, uint32_t lds_addr) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voffset), "s"(rsrc), "s"(lds_addr));
}

// The same copy marked non-temporal (nt): for data read exactly once, such as a decode's
// K/V cache. The line is not kept in the caches for reuse, which lifts a pure stream from
// about 6.0 to about 7.0 TB/s on gfx950; data that other workgroups read again (the tiled
// forward's K/V) keeps the default policy.
__device__ __forceinline__ void lds_copy16_stream(i32x4 rsrc, uint32_t voffset, uint32_t lds_addr) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voffset), "s"(rsrc), "s"(lds_addr));
}

// Raw buffer descriptor (stride 0, bounds-checked by num_records bytes).
__device__ __forceinline__ i32x4 buffer_desc(const void* base, int num_records) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), num_records, (int)kBufferFlags};
}
#endif  // __HIP_DEVICE_COMPILE__

}  // namespace aule
