// Row arithmetic shared by the staged kernels and the persistent kernel.
#pragma once

#include "common.h"

namespace moe {

// Combine + final weighted fusion of 8 columns (16-byte chunk c) of token t:
// out[t] = sum_j w[t,j] y[inv[t*k+j]] (+ ys[t]), fp32 fused multiply-adds in
// ascending j, rounded to bf16 once.
__device__ __forceinline__ void combine8(const uint16_t *y, const float *w, const int32_t *inv,
                                         const uint16_t *ys, uint16_t *out, int t, int c, int k,
                                         int HC) {
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; j++) {
    const int f = t * k + j;
    const float wj = w[f];
    float v[8];
    unpack8(((const uint4 *)y)[(size_t)inv[f] * HC + c], v);
#pragma unroll
    for (int q = 0; q < 8; q++) acc[q] = fmaf(wj, v[q], acc[q]);
  }
  if (ys) {
    float v[8];
    unpack8(((const uint4 *)ys)[(size_t)t * HC + c], v);
#pragma unroll
    for (int q = 0; q < 8; q++) acc[q] += v[q];
  }
  ((uint4 *)out)[(size_t)t * HC + c] = pack8(acc);
}

}  // namespace moe
