// Row arithmetic shared by the staged kernels and the persistent kernel.
#pragma once

#include "common.h"

namespace moe {

constexpr int kCombineMaxK = 16;  // top-k bound of the library

// Combine + final weighted fusion of 8 columns (16-byte chunk c) of token t:
// out[t] = sum_j w[t,j] y[inv[t*k+j]] (+ ys[t]), fp32 fused multiply-adds in
// ascending j, rounded to bf16 once.  All k rows' chunks are loaded before
// the first multiply-add, so one memory round trip covers the token.
// KMAX bounds k (8 or kCombineMaxK): the per-slot arrays take KMAX registers
// each, so the k <= 8 instantiation runs with far fewer registers (more
// waves in flight); the arithmetic is the same for every KMAX >= k.
template <int KMAX = kCombineMaxK>
__device__ __forceinline__ void combine8(const uint16_t *y, const float *w, const int32_t *inv,
                                         const uint16_t *ys, uint16_t *out, int t, int c, int k,
                                         int HC) {
  // row indices and weights first, unconditionally (slots past k repeat the
  // last one), so their loads issue together rather than one per row load
  int row[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    row[j] = inv[t * k + min(j, k - 1)];
    wt[j] = w[t * k + min(j, k - 1)];
  }
  // (needed here: keeps the compiler from sinking each index load next to
  // its row load)
#pragma unroll
  for (int j = 0; j < KMAX; j++) asm volatile("" ::"v"(row[j]));
  uint4 rv[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++)
    if (j < k) rv[j] = ld_once((const uint4 *)y + (size_t)row[j] * HC + c);  // read once
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    if (j < k) {
      const float wj = wt[j];
      float v[8];
      unpack8(rv[j], v);
#pragma unroll
      for (int q = 0; q < 8; q++) acc[q] = fmaf(wj, v[q], acc[q]);
    }
  }
  if (ys) {
    float v[8];
    unpack8(((const uint4 *)ys)[(size_t)t * HC + c], v);
#pragma unroll
    for (int q = 0; q < 8; q++) acc[q] += v[q];
  }
  // the layer's output is not read again by the layer: stored non-temporally
  st_once((uint4 *)out + (size_t)t * HC + c, pack8(acc));
}

}  // namespace moe
