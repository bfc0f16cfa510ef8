// The per-row FP8 encoding shared by the FP8 row kernels and the fused FP8 decode
// step's scoring launch, so that both write the same codes for the same row: a row's
// values are stored as OCP E4M3 codes of x * 2^-e (nearest, ties to even) with e the
// smallest exponent >= -126 for which the row's largest magnitude times 2^-e is at
// most 448, kept as the byte e + 127.
#pragma once
#include "se_internal.hpp"
#include "mfma_util.hpp"

namespace se {

// Smallest e >= -126 with amax * 2^-e <= 448 (0 for amax == 0).
__device__ __forceinline__ int fp8_row_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = frexpf(amax, &E);          // amax = m 2^E, m in [0.5, 1)
  // amax 2^-(E - 9) = 2m 2^8 lies in [256, 512): it fits iff 2m <= 1.75
  return max(E - 9 + (m > 0.875f ? 1 : 0), -126);
}

// Nearest E4M3 code of x 2^-e, ties to even (|x| 2^-e <= 448 by the choice of e).
__device__ __forceinline__ uint32_t fp8_encode(float x, int e) {
  const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = ldexpf(fabsf(x), -e);      // exact for every magnitude that can round above zero
  uint32_t mag;
  if (a < 0.015625f) {                       // below 2^-6: subnormal codes m 2^-9 (m = 8 is 0x08, the smallest normal)
    mag = uint32_t(__builtin_rintf(a * 512.f));
  } else {
    const uint32_t u = __float_as_uint(a);
    uint32_t t = u >> 20;                    // biased exponent and the top 3 mantissa bits
    const uint32_t rem = u & 0xfffffu;
    t += (rem > 0x80000u || (rem == 0x80000u && (t & 1u))) ? 1u : 0u;   // a carry moves into the exponent
    mag = t - (120u << 3);                   // exponent bias 127 -> 7
  }
  return sgn | mag;
}

// Stored value of code byte SEL of w, times 2^e, as fp32 (exact).
template <int SEL>
__device__ __forceinline__ float fp8_value(uint32_t w, int e) {
  return ldexpf(__builtin_amdgcn_cvt_f32_fp8(int(w), SEL), e);
}

// Quantizes the 8 bf16 values in `x` (one thread's part of a row of TPR threads) and
// returns their codes; `e` receives the row's exponent.
template <int TPR>
__device__ __forceinline__ uint2 fp8_quantize8(const u32x4 x, int& e) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(x[j]); v[2 * j + 1] = bf16_hi(x[j]); }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  e = fp8_row_exp(amax);
  uint2 c;
  c.x = fp8_encode(v[0], e) | fp8_encode(v[1], e) << 8 | fp8_encode(v[2], e) << 16 | fp8_encode(v[3], e) << 24;
  c.y = fp8_encode(v[4], e) | fp8_encode(v[5], e) << 8 | fp8_encode(v[6], e) << 16 | fp8_encode(v[7], e) << 24;
  return c;
}

}  // namespace se
