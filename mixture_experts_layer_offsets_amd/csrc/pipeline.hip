// Kernels of the minibatch-pipelined layer (the schedule itself is enqueued
// by api.hip on a communication stream and two GEMM streams).
//
// Source: kucoin.com news flash "O MoK do Cursor alcança aumento de
// desempenho de 2,37x no NVIDIA GB300 NVL72", §02: the layer's rows go to the
// experts in minibatches, so that the exchange of one minibatch overlaps the
// expert computation of another; the compute units are split between the
// exchange and the GEMMs, and stage completion is signalled on the GPU, with
// no host round trip per minibatch.  noticiai.com.br ("As três decisões de
// design que fazem a diferença") adds that the backward walks the minibatches
// in reverse.
//
// A minibatch is a range of MB expert-sorted rows [m*MB, min(R, (m+1)*MB)).
// Its row ranges are fixed by MB alone; only the split of a minibatch among
// experts and which tokens finish in it depend on the routing, and this plan
// kernel derives both on the GPU from the layout.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "mx_device.h"
#include "rows.h"

namespace moe {

// ---------------------------------------------------------------------------
// Plan, in two kernels (one workgroup of 1024 threads each), so that the
// GEMMs wait only for the first:
//   offsets: moff[m][e] = offsets[e] clamped to minibatch m's row range (so
//            expert e owns rows [moff[m][e], moff[m][e+1]) of minibatch m);
//            mts[m][e] = prefix of the 256-row tiles of those ranges (the
//            grouped GEMM's tile_start for minibatch m);
//   lists:   tl / tl_off: tokens grouped by the minibatch holding their LAST
//            routed row (last = 1: the forward combines a token once that
//            minibatch's down projection is done) or their FIRST routed row
//            (last = 0: the reverse walk has all of a token's row gradients
//            once that minibatch is done).
// The order of tokens inside one list is not fixed (LDS atomics place them);
// each token's result is computed on its own, so outputs do not depend on it.

__global__ __launch_bounds__(1024) void pipe_offsets_kernel(const int32_t *__restrict__ offsets,
                                                            int E, int R, int MB, int NM,
                                                            int32_t *__restrict__ moff,
                                                            int32_t *__restrict__ mts) {
  for (int m = threadIdx.x; m < NM; m += 1024) {
    const int lo = m * MB, hi = min(R, lo + MB);
    int32_t *mo = moff + (size_t)m * (E + 1), *mt = mts + (size_t)m * (E + 1);
    int tiles = 0;
    int prev = min(max(offsets[0], lo), hi);
    mo[0] = prev;
    for (int e = 0; e < E; e++) {
      const int nxt = min(max(offsets[e + 1], lo), hi);
      mo[e + 1] = nxt;
      mt[e] = tiles;
      tiles += (nxt - prev + kTileM - 1) / kTileM;
      prev = nxt;
    }
    mt[E] = tiles;
  }
}

__global__ __launch_bounds__(1024) void pipe_lists_kernel(const int32_t *__restrict__ inv, int T,
                                                          int k, int R, int MB, int NM, int last,
                                                          int32_t *__restrict__ tl,
                                                          int32_t *__restrict__ tl_off) {
  __shared__ int cnt[kPipeMaxMinibatches], base[kPipeMaxMinibatches];
  const int tid = threadIdx.x;
  for (int m = tid; m < NM; m += 1024) cnt[m] = 0;
  __syncthreads();
  auto key = [&](int t) {
    int hi = 0, lo = R;
    for (int j = 0; j < k; j++) {
      const int r = inv[t * k + j];
      hi = max(hi, r);
      lo = min(lo, r);
    }
    return (last ? hi : lo) / MB;
  };
  for (int t = tid; t < T; t += 1024) atomicAdd(&cnt[key(t)], 1);
  __syncthreads();
  if (tid == 0) {
    int sum = 0;
    for (int m = 0; m < NM; m++) { base[m] = sum; sum += cnt[m]; }
  }
  __syncthreads();
  for (int m = tid; m <= NM; m += 1024)
    tl_off[m] = m < NM ? base[m] : base[NM - 1] + cnt[NM - 1];
  __syncthreads();  // the offsets are read from base before placement moves it
  for (int t = tid; t < T; t += 1024) tl[atomicAdd(&base[key(t)], 1)] = t;
}

void launch_pipe_offsets(const int32_t *offsets, int E, int R, int MB, int NM, int32_t *moff,
                         int32_t *mts, hipStream_t s) {
  hipLaunchKernelGGL(pipe_offsets_kernel, dim3(1), dim3(1024), 0, s, offsets, E, R, MB, NM, moff,
                     mts);
}

void launch_pipe_lists(const int32_t *inv, int T, int k, int R, int MB, int NM, bool last,
                       int32_t *tl, int32_t *tl_off, hipStream_t s) {
  hipLaunchKernelGGL(pipe_lists_kernel, dim3(1), dim3(1024), 0, s, inv, T, k, R, MB, NM,
                     last ? 1 : 0, tl, tl_off);
}

// ---------------------------------------------------------------------------
// Combine of the tokens in list m: the same per-token arithmetic as the
// whole-layer combine (combine8), so the output is bit-identical to it.
// Grid (chunk groups, gy); the y blocks stride over the list.

__global__ __launch_bounds__(128) void combine_list_kernel(
    const uint16_t *__restrict__ y, const float *__restrict__ w, const int32_t *__restrict__ inv,
    const uint16_t *__restrict__ ys, uint16_t *__restrict__ out, const int32_t *__restrict__ tl,
    const int32_t *__restrict__ tl_off, int m, int k, int HC) {
  const int c = blockIdx.x * 128 + threadIdx.x;
  if (c >= HC) return;
  const int end = tl_off[m + 1];
  for (int i = tl_off[m] + blockIdx.y; i < end; i += gridDim.y)
    combine8(y, w, inv, ys, out, tl[i], c, k, HC);
}

void launch_combine_list(const uint16_t *y, const float *w, const int32_t *inv,
                         const uint16_t *ys, uint16_t *out, const int32_t *tl,
                         const int32_t *tl_off, int m, int T, int k, int H, hipStream_t s) {
  const int HC = H / 8;
  if (T <= 0) return;
  const int gy = std::min(T, 2048);
  hipLaunchKernelGGL(combine_list_kernel, dim3((HC + 127) / 128, gy), dim3(128), 0, s, y, w, inv,
                     ys, out, tl, tl_off, m, k, HC);
}

// ---------------------------------------------------------------------------
// Reverse-combine of sorted rows [r0, r0 + rows): for row r of flat index
// f = perm[r] (token t = f / k), dy[r] = w[f] dout[t] and
// dw[f] = <dout[t], y[r]>.  One 256-thread block per row; each lane's chunks
// (lane, lane + 256, ...) and the final reduction follow the whole-layer
// reverse-combine exactly, so dy and dw are bit-identical to it (and with
// MXFP8 so are dY's codes and scales, written here as there).

template <bool MXQ>
__global__ __launch_bounds__(256) void reverse_combine_rows_kernel(
    const uint4 *__restrict__ dout, const uint4 *__restrict__ y, const float *__restrict__ w,
    const int32_t *__restrict__ perm, uint4 *__restrict__ dy, float *__restrict__ dw, int r0,
    int k, int HC, uint2 *__restrict__ dyq, uint8_t *__restrict__ dys, long rows_total) {
  __shared__ float red[4];
  const int r = r0 + blockIdx.x, tid = threadIdx.x;
  const int f = perm[r], t = f / k;
  const float wt = w[f];
  float part = 0.0f;
  // four chunks per lane per pass, loads first; the dot product still
  // accumulates chunk by chunk in ascending column order
  for (int c0 = tid; c0 < HC; c0 += 1024) {
    uint4 dv[4], yv[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = c0 + 256 * u;
      if (c < HC) {
        dv[u] = ld_once(dout + (size_t)t * HC + c);
        yv[u] = ld_once(y + (size_t)r * HC + c);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = c0 + 256 * u;
      if (c < HC) {
        float d[8], v[8], o[8];
        unpack8(dv[u], d);
        unpack8(yv[u], v);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; q++) {
          s = fmaf(d[q], v[q], s);
          o[q] = wt * d[q];
        }
        part += s;
        const uint4 pk = pack8(o);
        dy[(size_t)r * HC + c] = pk;
        if constexpr (MXQ) {  // a quad's lanes share u and the guard
          float vq[8];
          unpack8(pk, vq);
          mx_put_chunk(vq, r, c, HC, rows_total, dyq, dys);
        }
      }
    }
  }
  const float s = wave_sum(part);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0 && dw) dw[f] = (red[0] + red[1]) + (red[2] + red[3]);
}

void launch_reverse_combine_rows(const uint16_t *dout, const uint16_t *y, const float *w,
                                 const int32_t *perm, uint16_t *dy, float *dw, int r0, int rows,
                                 int k, int H, uint8_t *dyq, uint8_t *dys, long rows_total,
                                 hipStream_t s) {
  if (rows <= 0) return;
  if (dyq)
    hipLaunchKernelGGL(reverse_combine_rows_kernel<true>, dim3(rows), dim3(256), 0, s,
                       (const uint4 *)dout, (const uint4 *)y, w, perm, (uint4 *)dy, dw, r0, k,
                       H / 8, (uint2 *)dyq, dys, rows_total);
  else
    hipLaunchKernelGGL(reverse_combine_rows_kernel<false>, dim3(rows), dim3(256), 0, s,
                       (const uint4 *)dout, (const uint4 *)y, w, perm, (uint4 *)dy, dw, r0, k,
                       H / 8, (uint2 *)nullptr, (uint8_t *)nullptr, rows_total);
}

// ---------------------------------------------------------------------------
// Reverse-dispatch of the tokens in list m, with the router's selected-logit
// gradient dsel[t,j] = w_j (dw_j - sum_j' w_j' dw_j') formed here from dw
// (the whole-layer path forms it in reverse-combine; the sum is the same
// wave butterfly over lanes j < k, so the values are bit-identical) and
// written once per token for the router's weight gradient.
// dx[t] = sum_j dX[inv[t*k+j]] + sum_j dsel[t,j] WrT[idx[t,j]] (+ dxs[t]).

__global__ __launch_bounds__(128) void reverse_dispatch_list_kernel(
    const uint4 *__restrict__ dX, const int32_t *__restrict__ inv, const int32_t *__restrict__ idx,
    const float *__restrict__ w, const float *__restrict__ dw, float *__restrict__ dsel,
    const uint4 *__restrict__ wrT, const uint4 *__restrict__ dxs, uint4 *__restrict__ dx,
    const int32_t *__restrict__ tl, const int32_t *__restrict__ tl_off, int m, int k, int HC) {
  const int c = blockIdx.x * 128 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int end = tl_off[m + 1];
  for (int i = tl_off[m] + blockIdx.y; i < end; i += gridDim.y) {
    const int t = tl[i];
    float sj[kMaxTopKList];
    if (wrT) {
      // every lane takes part in the butterfly, also past the row's end
      const float wl = lane < k ? w[t * k + lane] : 0.0f;
      const float dl = lane < k ? dw[t * k + lane] : 0.0f;
      const float sum = wave_sum(wl * dl);
#pragma unroll
      for (int j = 0; j < kMaxTopKList; j++)
        sj[j] = j < k ? w[t * k + j] * (dw[t * k + j] - sum) : 0.0f;
      if (blockIdx.x == 0 && threadIdx.x < k) dsel[t * k + threadIdx.x] = wl * (dl - sum);
    }
    if (c >= HC) continue;
    int row[kMaxTopKList];
#pragma unroll
    for (int j = 0; j < kMaxTopKList; j++) row[j] = inv[t * k + min(j, k - 1)];
#pragma unroll
    for (int j = 0; j < kMaxTopKList; j++) asm volatile("" ::"v"(row[j]));
    uint4 rv[kMaxTopKList];
#pragma unroll
    for (int j = 0; j < kMaxTopKList; j++)
      if (j < k) rv[j] = ld_once(dX + (size_t)row[j] * HC + c);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kMaxTopKList; j++) {
      if (j < k) {
        float v[8];
        unpack8(rv[j], v);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[q] += v[q];
      }
    }
    if (wrT) {
      for (int j = 0; j < k; j++) {
        float v[8];
        unpack8(wrT[(size_t)idx[t * k + j] * HC + c], v);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[q] = fmaf(sj[j], v[q], acc[q]);
      }
    }
    if (dxs) {
      float v[8];
      unpack8(dxs[(size_t)t * HC + c], v);
#pragma unroll
      for (int q = 0; q < 8; q++) acc[q] += v[q];
    }
    st_once((uint4 *)dx + (size_t)t * HC + c, pack8(acc));  // not read again by the layer
  }
}

void launch_reverse_dispatch_list(const uint16_t *dX, const int32_t *inv, const int32_t *idx,
                                  const float *w, const float *dw, float *dsel,
                                  const uint16_t *wrT, const uint16_t *dxs, uint16_t *dx,
                                  const int32_t *tl, const int32_t *tl_off, int m, int T, int k,
                                  int H, hipStream_t s) {
  const int HC = H / 8;
  if (T <= 0) return;
  const int gy = std::min(T, 2048);
  hipLaunchKernelGGL(reverse_dispatch_list_kernel, dim3((HC + 127) / 128, gy), dim3(128), 0, s,
                     (const uint4 *)dX, inv, idx, w, dw, dsel, (const uint4 *)wrT,
                     (const uint4 *)dxs, (uint4 *)dx, tl, tl_off, m, k, HC);
}

}  // namespace moe
