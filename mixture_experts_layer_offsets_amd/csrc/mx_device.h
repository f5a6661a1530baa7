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

__device__ __forceinline__ int floor_log2(float a) {  // a > 0
  const uint32_t u = __float_as_uint(a);
  const int ex = (int)(u >> 23);
  if (ex) return ex - 127;
  return -149 + (31 - __clz(u & 0x7FFFFFu));
}

}  // namespace moe
