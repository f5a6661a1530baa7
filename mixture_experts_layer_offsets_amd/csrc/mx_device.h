// MXFP8 element and scale conversions on the device (E4M3 codes, E8M0
// scales per 32 values; see permute.hip for the block rule).
#pragma once

#include "common.h"

namespace moe {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int floor_log2(float a) {  // a > 0
  const uint32_t u = __float_as_uint(a);
  const int ex = (int)(u >> 23);
  if (ex) return ex - 127;
  return -149 + (31 - __clz(u & 0x7FFFFFu));
}

// E8M0 exponent of a block from its largest magnitude: the element format's
// largest power of two (2^8 for E4M3) is lined up with amax's, clamped to the
// scale's range; an all-zero block takes the smallest scale.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int s = floor_log2(amax) - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// Four values to four E4M3 codes (one little-endian dword) at scale 2^s:
// each is scaled by 2^-s, clamped to +-448 and rounded to nearest even by the
// packed fp8 conversion.  The sign of a code is that of the value: adding
// +0.0 first turns -0.0 into +0.0, while a negative value whose scaled form
// underflows keeps its sign (-0.0, code 0x80).  With deq, the values the
// codes stand for (times 2^s) are written there.
__device__ __forceinline__ uint32_t e4m3_pack4(const float *x, int s, float *deq) {
  float sc[4];
#pragma unroll
  for (int b = 0; b < 4; b++) sc[b] = fminf(fmaxf(ldexpf(x[b] + 0.0f, -s), -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sc[0], sc[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sc[2], sc[3], w, true);
  if (deq) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    deq[0] = ldexpf(lo.x, s);
    deq[1] = ldexpf(lo.y, s);
    deq[2] = ldexpf(hi.x, s);
    deq[3] = ldexpf(hi.y, s);
  }
  return (uint32_t)w;
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
  const int s = mx_scale_exp(amax);
#pragma unroll
  for (int q = 0; q < 8; q++) w[q] = e4m3_pack4(v + 4 * q, s, deq ? deq + 4 * q : nullptr);
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
  const int s = mx_scale_exp(quad_max(amax));
  const uint32_t w0 = e4m3_pack4(v, s, deq);
  const uint32_t w1 = e4m3_pack4(v + 4, s, deq ? deq + 4 : nullptr);
  *codes = make_uint2(w0, w1);
  return (uint32_t)(s + 127);
}

// One 8-value chunk of a row in the row quantiser's output form (the four
// lanes of a quad hold one 32-value block and must all be active): E4M3
// codes at chunk c of row `row` (HC chunks per row), the block's E8M0 scale
// K-blocked, block b = c/4 at byte (b/4 * rows_total + row) * 4 + b%4.
__device__ __forceinline__ void mx_put_chunk(const float *v, long row, int c, int HC,
                                             long rows_total, uint2 *q, uint8_t *s) {
  uint2 codes;
  const uint32_t sc = mx_quad8(v, &codes, nullptr);
  q[(size_t)row * HC + c] = codes;
  if ((c & 3) == 0) s[((size_t)(c >> 4) * rows_total + row) * 4 + ((c >> 2) & 3)] = (uint8_t)sc;
}

}  // namespace moe
