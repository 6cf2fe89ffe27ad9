// Per-row quantisers of the 8-bit KV caches, shared by the KV write and the
// decode launch that appends each sequence's newest token.
//
// int8 follows KVCacheQuantizer.quantize's per_channel branch in the
// discosf.com article "KV Cache 优化与显存管理", section "三、实现示例":
// scale = absmax / 127 in fp32 (zero -> 1.0), code = clip(round-half-even(
// x / scale), -128, 127), fp32 IEEE division.  FP8 (OCP E4M3, the other
// 8-bit precision section "二、优化方向" names) applies the same per-row
// rule with E4M3's largest finite value: scale = absmax / 448, code = the
// E4M3 value nearest to x / scale, ties to the even code, saturating at
// +-448.
#pragma once

#include "pa_internal.h"

namespace pa {

// Nearest OCP E4M3 code to a finite fp32 value: ties to the even code,
// magnitudes at or above 448 saturate to 448 (0x7E); the sign bit is y's.
__device__ __forceinline__ uint8_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (!(a < 448.0f)) {
    mag = 0x7E;
  } else if (a < 0.015625f) {
    // below the smallest normal 2^-6 the codes are the multiples of 2^-9
    // (8 * 2^-9 is the smallest normal, code 0x08)
    mag = (uint32_t)rintf(a * 512.0f);
  } else {
    const uint32_t au = u & 0x7FFFFFFFu;
    uint32_t e = (au >> 23) - 127u + 7u;     // biased E4M3 exponent, 1 .. 15
    uint32_t m = (au >> 20) & 7u;            // top three mantissa bits
    const uint32_t rest = au & 0xFFFFFu;     // the 20 bits dropped
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) {
      if (++m == 8u) {
        m = 0;
        ++e;
      }
    }
    mag = (e << 3) | m;
    if (mag > 0x7Eu) mag = 0x7E;
  }
  return (uint8_t)(sign | mag);
}

// Codes of one (token, kv head) row held by a whole wave, PER values per
// lane; returns the row's scale (every lane).  FP8 = false: int8 codes.
template <int PER, bool FP8>
__device__ __forceinline__ float quantise_vals(const float (&x)[PER], uint8_t (&code)[PER]) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float s = __fdiv_rn(amax, FP8 ? 448.0f : 127.0f);
  s = (s > 0.f) ? s : 1.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float y = __fdiv_rn(x[e], s);
    if constexpr (FP8) {
      code[e] = e4m3_code(y);
    } else {
      const float qv = fminf(fmaxf(rintf(y), -128.f), 127.f);
      code[e] = (uint8_t)(int8_t)(int)qv;
    }
  }
  return s;
}

// Value of one code (exact in fp32).
template <bool FP8>
__device__ __forceinline__ float code_value(uint8_t c) {
  if constexpr (FP8) return __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false)[0];
  else return (float)(int8_t)c;
}

}  // namespace pa
