// MFMA helpers (gfx950): v_mfma_f32_16x16x32_bf16 and bf16 packing.
//
// Operand layout of the 16x16x32 bf16 MFMA used throughout (lane l, g = l / 16,
// c = l % 16): A lane l holds row c, k = 8g..8g+7; B lane l holds column c,
// k = 8g..8g+7; the 16x16 fp32 result lane l holds rows 4g..4g+3 of column c.
// Any permutation of k applied to both A and B leaves the product unchanged,
// which the kernels use to give each lane contiguous 64-byte row reads.
#pragma once
#include "se_internal.hpp"

namespace se {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bf16 pair (lo, hi) from two fp32 values, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ float bf16x2_lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16x2_hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value {hi_src : lo_src}.
// Low halves of two words: {lo16(a), lo16(b)}; high halves: {hi16(a), hi16(b)}.
__device__ __forceinline__ uint32_t lo16_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi16_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }


}  // namespace se
