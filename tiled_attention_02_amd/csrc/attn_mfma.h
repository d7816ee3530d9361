// gfx950 matrix-core helpers shared by the forward and backward kernels: operand vector
// types, the 32x32x16 bf16/fp16 MFMA with its pack / dot helpers, and the row permutation
// sigma that makes a product's accumulator registers the operand of the next product.
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

}  // namespace aule
