// Data movement of the layer: dispatch, combine and their backward mirrors,
// plus the router's weight gradient and weight packing.
//
// Sources: kucoin.com news flash "O MoK do Cursor alcança aumento de
// desempenho de 2,37x no NVIDIA GB300 NVL72":
//   §01  dispatch sends each token to its experts, combine returns every
//        result to the token's original position; training adds two rounds
//        in the opposite direction;
//   §02  the destination pulls the rows it needs knowing only where each
//        sits in the source (pull dispatch), results are pushed back to their
//        known origin (push combine); the backward uses pull reverse-combine
//        and push reverse-dispatch; MXFP8 activation quantisation is fused
//        into dispatch;
//   §03  the measured layer ends with the final weighted fusion.
// On one GPU the "exchange" is an HBM gather or scatter: every kernel here
// moves whole rows with 16-byte accesses, reads each source row once per use
// and reduces in a fixed order.
#include "common.h"
#include "kernels.h"
#include "mx_device.h"
#include "rows.h"

namespace moe {

// ---------------------------------------------------------------------------
// Dispatch.  One wave per sorted row r copies token perm[r] / k.  Each lane
// issues up to kCopyBatch 16-byte loads before its first store, so a wave
// keeps a whole batch of the row in flight instead of one chunk per memory
// round trip.

constexpr int kCopyBatch = 8;
constexpr int kMaxTopKPush = 16;  // top-k bound of the library

__global__ __launch_bounds__(256) void dispatch_bf16_kernel(const uint4 *__restrict__ x,
                                                            const int32_t *__restrict__ perm,
                                                            uint4 *__restrict__ xp, int R, int k,
                                                            int HC) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const uint4 *src = x + (size_t)(perm[r] / k) * HC;
  uint4 *dst = xp + (size_t)r * HC;
  for (int c0 = threadIdx.x & 63; c0 < HC; c0 += 64 * kCopyBatch) {
    // loads past the row's end re-read its last chunk (kept in registers,
    // not stored), so the batch needs no predicated loads
    uint4 v[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; u++) v[u] = src[min(c0 + 64 * u, HC - 1)];
    // the values are needed here, so the compiler cannot sink each load into
    // its (predicated) store's block, one round trip per chunk
#pragma unroll
    for (int u = 0; u < kCopyBatch; u++)
      asm volatile("" ::"v"(v[u].x), "v"(v[u].y), "v"(v[u].z), "v"(v[u].w));
#pragma unroll
    for (int u = 0; u < kCopyBatch; u++)
      if (c0 + 64 * u < HC) dst[c0 + 64 * u] = v[u];
  }
}

void launch_dispatch_bf16(const uint16_t *x, const int32_t *perm, uint16_t *xp, int R, int k,
                          int H, hipStream_t s) {
  if (R <= 0) return;
  hipLaunchKernelGGL(dispatch_bf16_kernel, dim3((R + 3) / 4), dim3(256), 0, s,
                     (const uint4 *)x, perm, (uint4 *)xp, R, k, H / 8);
}

// MX dispatch: each lane converts 8 consecutive values (one 16-byte load),
// four lanes of a quad form one 32-value block (block maximum by two DPP
// exchanges), so loads and stores are contiguous across the wave.  Writes the
// E4M3 codes, the E8M0 scales and (if xhat) the dequantised row as bf16.
// The grid covers whole quads: R * H/8 is a multiple of 4.
// Rows [row0, row0 + R) of an output of `rows_total` rows (the scale plane's
// row stride), so one minibatch of sorted rows can be converted on its own.
__global__ __launch_bounds__(256) void dispatch_mx_kernel(
    const uint4 *__restrict__ x, const int32_t *__restrict__ perm, uint2 *__restrict__ xq,
    uint8_t *__restrict__ xs, uint4 *__restrict__ xhat, int row0, int R, long rows_total, int k,
    int HC /* H/8 */) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long)R * HC) return;
  const int r = row0 + (int)(id / HC), c = (int)(id - (long)(r - row0) * HC);
  const int src_row = perm ? perm[r] / k : r;
  float v[8];
  unpack8(x[(size_t)src_row * HC + c], v);
  uint2 codes;
  float deq[8];
  const uint32_t sc = mx_quad8(v, &codes, deq);
  xq[(size_t)r * HC + c] = codes;
  // scales K-blocked: block b = c/4 of row r at byte (b/4 * rows_total + r) * 4 + b%4
  if ((c & 3) == 0) xs[((size_t)(c >> 4) * rows_total + r) * 4 + ((c >> 2) & 3)] = (uint8_t)sc;
  if (xhat) xhat[(size_t)r * HC + c] = pack8(deq);
}

void launch_dispatch_mx_range(const uint16_t *x, const int32_t *perm, uint8_t *xq, uint8_t *xs,
                              uint16_t *xhat, int row0, int rows, int rows_total, int k, int H,
                              hipStream_t s) {
  const long n = (long)rows * (H / 8);
  if (n <= 0) return;
  hipLaunchKernelGGL(dispatch_mx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const uint4 *)x, perm, (uint2 *)xq, xs, (uint4 *)xhat, row0, rows,
                     (long)rows_total, k, H / 8);
}

void launch_dispatch_mx(const uint16_t *x, const int32_t *perm, uint8_t *xq, uint8_t *xs,
                        uint16_t *xhat, int R, int k, int H, hipStream_t s) {
  launch_dispatch_mx_range(x, perm, xq, xs, xhat, 0, R, R, k, H, s);
}

// Dispatch in scatter form, for the layer (which has inv = perm^-1): token
// t's row is read -- and with MXFP8 quantised -- once, then written to its k
// sorted rows inv[t*k + j].  Same result as the gather above; it reads each
// token once instead of k times.  Grid (H/8 chunks over 128 threads, T).

// Only rows in [r0, r1) are written (one minibatch of sorted rows; RANGE =
// false is the whole set [0, T*k) and carries no test).  KMAX bounds k (8 or
// kMaxTopKPush): no index loads past the bound.  The token's chunk is loaded
// before the row indices resolve (it is in bounds either way), so its load
// overlaps theirs instead of waiting for a test that depends on them.
template <int KMAX, bool RANGE>
__global__ __launch_bounds__(128) void dispatch_push_bf16_kernel(const uint4 *__restrict__ x,
                                                                 const int32_t *__restrict__ inv,
                                                                 uint4 *__restrict__ xp, int k,
                                                                 int HC, int r0, int r1) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 128 + threadIdx.x;
  if (c >= HC) return;
  const uint4 v = ld_once(x + (size_t)t * HC + c);
  int row[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) row[j] = inv[t * k + min(j, k - 1)];
#pragma unroll
  for (int j = 0; j < KMAX; j++)
    if (j < k && (!RANGE || (row[j] >= r0 && row[j] < r1))) xp[(size_t)row[j] * HC + c] = v;
}

void launch_dispatch_push_bf16_range(const uint16_t *x, const int32_t *inv, uint16_t *xp, int T,
                                     int k, int H, int r0, int r1, hipStream_t s) {
  const int HC = H / 8;
  if (T <= 0) return;
  const dim3 g((HC + 127) / 128, T), b(128);
  const bool all = r0 <= 0 && r1 >= T * k;
  if (k <= 8 && all)
    hipLaunchKernelGGL((dispatch_push_bf16_kernel<8, false>), g, b, 0, s, (const uint4 *)x, inv,
                       (uint4 *)xp, k, HC, r0, r1);
  else if (k <= 8)
    hipLaunchKernelGGL((dispatch_push_bf16_kernel<8, true>), g, b, 0, s, (const uint4 *)x, inv,
                       (uint4 *)xp, k, HC, r0, r1);
  else if (all)
    hipLaunchKernelGGL((dispatch_push_bf16_kernel<kMaxTopKPush, false>), g, b, 0, s,
                       (const uint4 *)x, inv, (uint4 *)xp, k, HC, r0, r1);
  else
    hipLaunchKernelGGL((dispatch_push_bf16_kernel<kMaxTopKPush, true>), g, b, 0, s,
                       (const uint4 *)x, inv, (uint4 *)xp, k, HC, r0, r1);
}

void launch_dispatch_push_bf16(const uint16_t *x, const int32_t *inv, uint16_t *xp, int T, int k,
                               int H, hipStream_t s) {
  launch_dispatch_push_bf16_range(x, inv, xp, T, k, H, 0, T * k, s);
}

// MX: each lane quantises 8 values as in dispatch_mx_kernel (a quad of lanes
// per 32-value block), then stores codes, scale and round trip to k rows.
// Only rows in [r0, r1) are written (RANGE = false: all rows, no test).
// Every lane of a quad (one token's 32-value block) runs the conversion, so
// the quad's block-maximum exchange always has all four lanes; the token's
// chunk is loaded before the row indices resolve.  KMAX bounds k.
template <int KMAX, bool RANGE>
__global__ __launch_bounds__(256) void dispatch_push_mx_kernel(
    const uint4 *__restrict__ x, const int32_t *__restrict__ inv, uint2 *__restrict__ xq,
    uint8_t *__restrict__ xs, uint4 *__restrict__ xhat, int T, int k, int HC /* H/8 */, int r0,
    int r1) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long)T * HC) return;
  const long R = (long)T * k;  // rows of the output (scale plane stride)
  const int t = (int)(id / HC), c = (int)(id - (long)t * HC);
  float v[8];
  unpack8(ld_once(x + (size_t)t * HC + c), v);
  int row[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) row[j] = inv[t * k + min(j, k - 1)];
  uint2 codes;
  float deq[8];
  const uint32_t sc = mx_quad8(v, &codes, deq);
  const uint4 hat = pack8(deq);
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    if (j < k && (!RANGE || (row[j] >= r0 && row[j] < r1))) {
      const size_t r = (size_t)row[j];
      xq[r * HC + c] = codes;
      if ((c & 3) == 0) xs[((size_t)(c >> 4) * R + r) * 4 + ((c >> 2) & 3)] = (uint8_t)sc;
      // the round trip is read only by the backward: stored non-temporally
      // so that it does not evict the codes the gate/up GEMM reads next
      if (xhat) st_once(xhat + r * HC + c, hat);
    }
  }
}

void launch_dispatch_push_mx_range(const uint16_t *x, const int32_t *inv, uint8_t *xq,
                                   uint8_t *xs, uint16_t *xhat, int T, int k, int H, int r0,
                                   int r1, hipStream_t s) {
  const long n = (long)T * (H / 8);
  if (n <= 0) return;
  const dim3 g((unsigned)((n + 255) / 256)), b(256);
  const bool all = r0 <= 0 && r1 >= T * k;
  auto *X = (const uint4 *)x;
  auto *Q = (uint2 *)xq;
  auto *Hh = (uint4 *)xhat;
  if (k <= 8 && all)
    hipLaunchKernelGGL((dispatch_push_mx_kernel<8, false>), g, b, 0, s, X, inv, Q, xs, Hh, T, k,
                       H / 8, r0, r1);
  else if (k <= 8)
    hipLaunchKernelGGL((dispatch_push_mx_kernel<8, true>), g, b, 0, s, X, inv, Q, xs, Hh, T, k,
                       H / 8, r0, r1);
  else if (all)
    hipLaunchKernelGGL((dispatch_push_mx_kernel<kMaxTopKPush, false>), g, b, 0, s, X, inv, Q, xs,
                       Hh, T, k, H / 8, r0, r1);
  else
    hipLaunchKernelGGL((dispatch_push_mx_kernel<kMaxTopKPush, true>), g, b, 0, s, X, inv, Q, xs,
                       Hh, T, k, H / 8, r0, r1);
}

void launch_dispatch_push_mx(const uint16_t *x, const int32_t *inv, uint8_t *xq, uint8_t *xs,
                             uint16_t *xhat, int T, int k, int H, hipStream_t s) {
  launch_dispatch_push_mx_range(x, inv, xq, xs, xhat, T, k, H, 0, T * k, s);
}

// Row-wise MX quantisation of a bf16 matrix along its contiguous axis.
void launch_quant_rows_mx(const uint16_t *src, int rows, int cols, uint8_t *q, uint8_t *sc,
                          hipStream_t s) {
  launch_dispatch_mx_range(src, nullptr, q, sc, nullptr, 0, rows, rows, 1, cols, s);
}

void launch_quant_rows_mx_range(const uint16_t *src, int row0, int rows, int rows_total, int cols,
                                uint8_t *q, uint8_t *sc, hipStream_t s) {
  launch_dispatch_mx_range(src, nullptr, q, sc, nullptr, row0, rows, rows_total, 1, cols, s);
}

// ---------------------------------------------------------------------------
// Combine + final weighted fusion: out[t] = sum_j w[t,j] y[inv[t*k+j]] (+ ys[t]),
// fp32 fused multiply-adds in ascending j.  Grid (chunk groups, T).

// One wave per block: measured on MI355X at the Kimi shape (after the cache
// is flushed), 64-thread blocks gather about 2 % faster than 128 or 256.
constexpr int kGatherBlock = 64;

template <int KMAX>
__global__ __launch_bounds__(kGatherBlock) void combine_kernel(const uint16_t *__restrict__ y,
                                                               const float *__restrict__ w,
                                                               const int32_t *__restrict__ inv,
                                                               const uint16_t *__restrict__ ys,
                                                               uint16_t *__restrict__ out, int k,
                                                               int HC) {
  const int c = blockIdx.x * kGatherBlock + threadIdx.x;
  if (c < HC) combine8<KMAX>(y, w, inv, ys, out, blockIdx.y, c, k, HC);
}

void launch_combine(const uint16_t *y, const float *w, const int32_t *inv, const uint16_t *ys,
                    uint16_t *out, int T, int k, int H, hipStream_t s) {
  const int HC = H / 8;
  if (T <= 0) return;
  const dim3 g((HC + kGatherBlock - 1) / kGatherBlock, T), b(kGatherBlock);
  if (k <= 8)
    hipLaunchKernelGGL(combine_kernel<8>, g, b, 0, s, y, w, inv, ys, out, k, HC);
  else
    hipLaunchKernelGGL(combine_kernel<kCombineMaxK>, g, b, 0, s, y, w, inv, ys, out, k, HC);
}

// ---------------------------------------------------------------------------
// Reverse-combine: each token's output gradient goes to its k rows scaled by
// the slot weight, and dw[t,j] = <dout[t], y[row]>.  With a router, also the
// selected-logit gradient dsel[t,j] = w_j (dw_j - sum_j' w_j' dw_j').
// One 256-thread block per token; the dot products reduce in a fixed tree.
// With MXFP8 (MXQ) each dY chunk is also written in the row quantiser's form
// (codes and K-blocked scales of the stored bf16 values), the down data
// gradient's operand, so dY is not read back to quantise it.

constexpr int kMaxTopK = 16;

// KMAX bounds k (see combine8): 8 for k <= 8, else kMaxTopK.
template <int KMAX, bool MXQ>
__global__ __launch_bounds__(256) void reverse_combine_kernel(
    const uint4 *__restrict__ dout, const uint4 *__restrict__ y, const float *__restrict__ w,
    const int32_t *__restrict__ inv, uint4 *__restrict__ dy, float *__restrict__ dw,
    float *__restrict__ dsel, int k, int HC, uint2 *__restrict__ dyq, uint8_t *__restrict__ dys,
    long rows_total) {
  __shared__ float red[KMAX][4];
  const int t = blockIdx.x, tid = threadIdx.x;
  float part[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) part[j] = 0.0f;
  int rows[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) {  // slots past k repeat the last one, unused
    rows[j] = inv[t * k + min(j, k - 1)];
    wt[j] = w[t * k + min(j, k - 1)];
  }
  // NCH chunks per lane per pass (two; one with MXQ, whose conversion
  // needs the registers), all of a pass's loads issued before its
  // arithmetic; partial dot products still accumulate chunk by chunk in
  // ascending column order, so dw is the same for either NCH.
  constexpr int NCH = MXQ ? 1 : 2;
  for (int c0 = tid; c0 < HC; c0 += 256 * NCH) {
    const bool has1 = NCH == 2 && c0 + 256 < HC;
    // dout and the k rows of y are each read once
    const uint4 d0 = ld_once(dout + (size_t)t * HC + c0);
    const uint4 d1 = has1 ? ld_once(dout + (size_t)t * HC + c0 + 256) : make_uint4(0, 0, 0, 0);
    uint4 yv[KMAX][2];
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
      if (j < k) {
        yv[j][0] = ld_once(y + (size_t)rows[j] * HC + c0);
        if (has1) yv[j][1] = ld_once(y + (size_t)rows[j] * HC + c0 + 256);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      if (u == 1 && !has1) break;
      const int c = c0 + 256 * u;
      float d[8];
      unpack8(u ? d1 : d0, d);
#pragma unroll
      for (int j = 0; j < KMAX; j++) {
        if (j < k) {
          float v[8], o[8];
          unpack8(yv[j][u], v);
          float s = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; q++) {
            s = fmaf(d[q], v[q], s);
            o[q] = wt[j] * d[q];
          }
          part[j] += s;
          const uint4 pk = pack8(o);
          dy[(size_t)rows[j] * HC + c] = pk;
          if constexpr (MXQ) {  // a quad's lanes share j, u and the guards
            float vq[8];
            unpack8(pk, vq);
            mx_put_chunk(vq, rows[j], c, HC, rows_total, dyq, dys);
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    if (j < k) {
      const float s = wave_sum(part[j]);
      if ((tid & 63) == 0) red[j][tid >> 6] = s;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const float dwj = tid < k ? (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]) : 0.0f;
    if (tid < k && dw) dw[t * k + tid] = dwj;
    if (dsel) {
      const float wj = tid < k ? w[t * k + tid] : 0.0f;
      const float sum = wave_sum(wj * dwj);
      if (tid < k) dsel[t * k + tid] = wj * (dwj - sum);
    }
  }
}

void launch_reverse_combine(const uint16_t *dout, const uint16_t *y, const float *w,
                            const int32_t *inv, uint16_t *dy, float *dw, float *dsel, int T,
                            int k, int H, uint8_t *dyq, uint8_t *dys, hipStream_t s) {
  if (T <= 0) return;
  const long R = (long)T * k;
  uint2 *q = (uint2 *)dyq;
  if (k <= 8 && dyq)
    hipLaunchKernelGGL((reverse_combine_kernel<8, true>), dim3(T), dim3(256), 0, s,
                       (const uint4 *)dout, (const uint4 *)y, w, inv, (uint4 *)dy, dw, dsel, k,
                       H / 8, q, dys, R);
  else if (k <= 8)
    hipLaunchKernelGGL((reverse_combine_kernel<8, false>), dim3(T), dim3(256), 0, s,
                       (const uint4 *)dout, (const uint4 *)y, w, inv, (uint4 *)dy, dw, dsel, k,
                       H / 8, q, dys, R);
  else if (dyq)
    hipLaunchKernelGGL((reverse_combine_kernel<kMaxTopK, true>), dim3(T), dim3(256), 0, s,
                       (const uint4 *)dout, (const uint4 *)y, w, inv, (uint4 *)dy, dw, dsel, k,
                       H / 8, q, dys, R);
  else
    hipLaunchKernelGGL((reverse_combine_kernel<kMaxTopK, false>), dim3(T), dim3(256), 0, s,
                       (const uint4 *)dout, (const uint4 *)y, w, inv, (uint4 *)dy, dw, dsel, k,
                       H / 8, q, dys, R);
}

// ---------------------------------------------------------------------------
// Reverse-dispatch: dx[t] = sum_j dX[inv[t*k+j]] + sum_j dsel[t,j] Wr^T[idx[t,j]]
// (+ dxs[t]), fp32 in ascending j, stored as bf16.

// KMAX bounds k (see combine8); ROUTER / SHARED: whether the router term and
// the shared expert's rows exist (the kernel without them carries neither
// branch nor their registers).
template <int KMAX, bool ROUTER, bool SHARED>
__global__ __launch_bounds__(kGatherBlock) void reverse_dispatch_kernel(
    const uint4 *__restrict__ dX, const int32_t *__restrict__ inv, const int32_t *__restrict__ idx,
    const float *__restrict__ dsel, const uint4 *__restrict__ wrT, const uint4 *__restrict__ dxs,
    uint4 *__restrict__ dx, int k, int HC) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * kGatherBlock + threadIdx.x;
  if (c >= HC) return;
  // all k row indices, then all k rows' chunks, in flight before the first
  // add (index slots past k repeat the last one)
  int row[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) row[j] = inv[t * k + min(j, k - 1)];
#pragma unroll
  for (int j = 0; j < KMAX; j++) asm volatile("" ::"v"(row[j]));  // materialise here
  uint4 rv[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++)
    if (j < k) rv[j] = ld_once(dX + (size_t)row[j] * HC + c);  // read once
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    if (j < k) {
      float v[8];
      unpack8(rv[j], v);
#pragma unroll
      for (int q = 0; q < 8; q++) acc[q] += v[q];
    }
  }
  if constexpr (ROUTER) {
    for (int j = 0; j < k; j++) {
      const float sj = dsel[t * k + j];
      float v[8];
      unpack8(wrT[(size_t)idx[t * k + j] * HC + c], v);
#pragma unroll
      for (int q = 0; q < 8; q++) acc[q] = fmaf(sj, v[q], acc[q]);
    }
  }
  if constexpr (SHARED) {
    float v[8];
    unpack8(dxs[(size_t)t * HC + c], v);
#pragma unroll
    for (int q = 0; q < 8; q++) acc[q] += v[q];
  }
  st_once(dx + (size_t)t * HC + c, pack8(acc));  // not read again by the layer
}

template <int KMAX>
static void launch_rd(const dim3 &g, const uint16_t *dX, const int32_t *inv, const int32_t *idx,
                      const float *dsel, const uint16_t *wrT, const uint16_t *dxs, uint16_t *dx,
                      int k, int HC, hipStream_t s) {
  const dim3 b(kGatherBlock);
  auto *X = (const uint4 *)dX;
  auto *W = (const uint4 *)wrT;
  auto *S = (const uint4 *)dxs;
  auto *D = (uint4 *)dx;
  if (wrT && dxs)
    hipLaunchKernelGGL((reverse_dispatch_kernel<KMAX, true, true>), g, b, 0, s, X, inv, idx, dsel,
                       W, S, D, k, HC);
  else if (wrT)
    hipLaunchKernelGGL((reverse_dispatch_kernel<KMAX, true, false>), g, b, 0, s, X, inv, idx,
                       dsel, W, S, D, k, HC);
  else if (dxs)
    hipLaunchKernelGGL((reverse_dispatch_kernel<KMAX, false, true>), g, b, 0, s, X, inv, idx,
                       dsel, W, S, D, k, HC);
  else
    hipLaunchKernelGGL((reverse_dispatch_kernel<KMAX, false, false>), g, b, 0, s, X, inv, idx,
                       dsel, W, S, D, k, HC);
}

void launch_reverse_dispatch(const uint16_t *dX, const int32_t *inv, const int32_t *idx,
                             const float *dsel, const uint16_t *wrT, const uint16_t *dxs,
                             uint16_t *dx, int T, int k, int H, hipStream_t s) {
  const int HC = H / 8;
  if (T <= 0) return;
  const dim3 g((HC + kGatherBlock - 1) / kGatherBlock, T);
  if (k <= 8)
    launch_rd<8>(g, dX, inv, idx, dsel, wrT, dxs, dx, k, HC, s);
  else
    launch_rd<kMaxTopK>(g, dX, inv, idx, dsel, wrT, dxs, dx, k, HC, s);
}

// ---------------------------------------------------------------------------
// Router weight gradient: dWr[h][e] = sum over expert e's rows of
// dsel[f] * x[f/k][h], rows in sorted (ascending) order.  Grid (H/2048, E).

__global__ __launch_bounds__(256) void router_wgrad_kernel(const uint4 *__restrict__ x,
                                                           const int32_t *__restrict__ perm,
                                                           const int32_t *__restrict__ offsets,
                                                           const float *__restrict__ dsel,
                                                           float *__restrict__ dwr, int E, int k,
                                                           int HC) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= HC) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int r1 = offsets[e + 1];
  for (int r = offsets[e]; r < r1; r++) {
    const int f = perm[r];
    const float s = dsel[f];
    float v[8];
    unpack8(x[(size_t)(f / k) * HC + c], v);
#pragma unroll
    for (int q = 0; q < 8; q++) acc[q] = fmaf(s, v[q], acc[q]);
  }
#pragma unroll
  for (int q = 0; q < 8; q++) dwr[(size_t)(c * 8 + q) * E + e] = acc[q];
}

void launch_router_wgrad(const uint16_t *x, const int32_t *perm, const int32_t *offsets,
                         const float *dsel, float *dwr, int E, int k, int H, hipStream_t s) {
  const int HC = H / 8;
  hipLaunchKernelGGL(router_wgrad_kernel, dim3((HC + 255) / 256, E), dim3(256), 0, s,
                     (const uint4 *)x, perm, offsets, dsel, dwr, E, k, HC);
}

// ---------------------------------------------------------------------------
// Weight packing.
// transpose_pack: out[g][map(c)][r] = in[g][r][c] for in [G][rows][cols],
//   map(c) = (c / 32) * blk_stride + blk_off + c % 32; out rows have `rows`
//   elements; out has out_rows_total rows per group.
// interleave_copy: out[g][r][map(c)] = in[g][r][c]; out rows have out_cols.

__global__ __launch_bounds__(256) void transpose_pack_kernel(const uint16_t *__restrict__ in,
                                                             uint16_t *__restrict__ out, int rows,
                                                             int cols, int out_rows_total,
                                                             int blk_stride, int blk_off) {
  __shared__ uint16_t tile[64][65];
  const int g = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t *src = in + (size_t)g * rows * cols;
  uint16_t *dst = out + (size_t)g * out_rows_total * rows;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i >> 6, cc = i & 63;
    if (r0 + rr < rows && c0 + cc < cols) tile[rr][cc] = src[(size_t)(r0 + rr) * cols + c0 + cc];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i >> 6, rr = i & 63;
    const int c = c0 + cc, r = r0 + rr;
    if (r < rows && c < cols) {
      const int orow = (c >> 5) * blk_stride + blk_off + (c & 31);
      dst[(size_t)orow * rows + r] = tile[rr][cc];
    }
  }
}

void launch_transpose_pack(const uint16_t *in, uint16_t *out, int G, int rows, int cols,
                           int out_rows_total, int blk_stride, int blk_off, hipStream_t s) {
  hipLaunchKernelGGL(transpose_pack_kernel, dim3((cols + 63) / 64, (rows + 63) / 64, G),
                     dim3(256), 0, s, in, out, rows, cols, out_rows_total, blk_stride, blk_off);
}

__global__ __launch_bounds__(256) void interleave_copy_kernel(const uint16_t *__restrict__ in,
                                                              uint16_t *__restrict__ out,
                                                              int rows, int cols, int out_cols,
                                                              int blk_stride, int blk_off) {
  const int g = blockIdx.z, r = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const int oc = (c >> 5) * blk_stride + blk_off + (c & 31);
  out[((size_t)g * rows + r) * out_cols + oc] = in[((size_t)g * rows + r) * cols + c];
}

void launch_interleave_copy(const uint16_t *in, uint16_t *out, int G, int rows, int cols,
                            int out_cols, int blk_stride, int blk_off, hipStream_t s) {
  hipLaunchKernelGGL(interleave_copy_kernel, dim3((cols + 255) / 256, rows, G), dim3(256), 0, s,
                     in, out, rows, cols, out_cols, blk_stride, blk_off);
}

}  // namespace moe
