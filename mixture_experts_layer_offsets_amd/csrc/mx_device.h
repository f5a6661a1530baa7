// MXFP8 element and scale conversions on the device (E4M3 codes, E8M0
// scales per 32 values; see permute.hip for the block rule).
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t e4m3_encode(float v, bool neg) {
  const float a = fabsf(v);
  const uint32_t sign = neg ? 0x80u : 0u;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);  // spacing 2^-9
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);  // round to 3 mantissa bits
  const int e = (int)(r >> 23) - 127;
  return sign | ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  const float mag = ex ? ldexpf((float)(8u + m), (int)ex - 10) : ldexpf((float)m, -9);
  return (c & 0x80u) ? -mag : mag;
}

// E4M3 code of a value with |v| <= 448 (sign bit from `neg`), and in `mag`
// the magnitude that code stands for (the rounded |v|).
__device__ __forceinline__ uint32_t e4m3_encode_mag(float v, bool neg, float *mag) {
  const float a = fabsf(v);
  const uint32_t sign = neg ? 0x80u : 0u;
  if (a < 0.015625f) {  // subnormal codes: spacing 2^-9
    const float q = rintf(a * 512.0f);
    *mag = q * 0.001953125f;
    return sign | (uint32_t)q;
  }
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
  *mag = __uint_as_float(r);
  const int e = (int)(r >> 23) - 127;
  return sign | ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ int floor_log2(float a) {  // a > 0
  const uint32_t u = __float_as_uint(a);
  const int ex = (int)(u >> 23);
  if (ex) return ex - 127;
  return -149 + (31 - __clz(u & 0x7FFFFFu));
}

// MXFP8 conversion of one block of 32 values (E4M3 elements, E8M0 scale):
//   s = clamp(floor(log2 amax) - 8, -127, 127), scale code s + 127,
//   code_i = E4M3(clamp(v_i * 2^-s, -448, 448)), nearest-even,
//   an all-zero block gets scale code 0 (and zero codes).
// Writes the 32 codes as 8 little-endian dwords to w, the dequantised values
// to deq (if not null), and returns the scale code.
__device__ __forceinline__ uint32_t mx_block32(const float *v, uint32_t *w, float *deq) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  int s = -127;
  if (amax > 0.0f) {
    s = floor_log2(amax) - 8;
    s = s < -127 ? -127 : (s > 127 ? 127 : s);
  }
#pragma unroll
  for (int q = 0; q < 8; q++) {
    uint32_t d = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const float x = v[q * 4 + b];
      const float sc = fminf(fmaxf(ldexpf(x, -s), -448.0f), 448.0f);
      float mag;
      const uint32_t c = e4m3_encode_mag(sc, x < 0.0f, &mag);
      d |= c << (8 * b);
      if (deq) deq[q * 4 + b] = ldexpf(x < 0.0f ? -mag : mag, s);
    }
    w[q] = d;
  }
  return (uint32_t)(s + 127);
}

// Maximum over the four lanes of a quad (DPP quad permutations; every lane
// of the quad must be active).
__device__ __forceinline__ float quad_max(float x) {
  int b = __float_as_int(x);
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));
  b = __float_as_int(x);
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false)));
  return x;
}

// The same conversion as mx_block32 with a block spread over the four lanes
// of a quad, 8 values per lane (lane q of the quad holds values 8q..8q+7).
// Returns the block's scale code in every lane of the quad.
__device__ __forceinline__ uint32_t mx_quad8(const float *v, uint2 *codes, float *deq) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
  amax = quad_max(amax);
  int s = -127;
  if (amax > 0.0f) {
    s = floor_log2(amax) - 8;
    s = s < -127 ? -127 : (s > 127 ? 127 : s);
  }
  uint32_t w[2];
#pragma unroll
  for (int q = 0; q < 2; q++) {
    uint32_t d = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const float x = v[q * 4 + b];
      const float sc = fminf(fmaxf(ldexpf(x, -s), -448.0f), 448.0f);
      float mag;
      const uint32_t c = e4m3_encode_mag(sc, x < 0.0f, &mag);
      d |= c << (8 * b);
      deq[q * 4 + b] = ldexpf(x < 0.0f ? -mag : mag, s);
    }
    w[q] = d;
  }
  *codes = make_uint2(w[0], w[1]);
  return (uint32_t)(s + 127);
}

}  // namespace moe
