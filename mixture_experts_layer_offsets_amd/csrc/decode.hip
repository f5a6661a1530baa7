// Few-token (decode) forward of the expert FFN.
//
// noticiai.com.br ("Cursor abre código do Mixture-of-Kittens ...") mentions a
// separate decode kernel for inference, where each token is handled by its
// own small group of threads.  With a handful of tokens the layer is bound by
// reading the selected experts' weights, not by arithmetic: a 256-row MFMA
// tile would stream the same weights while doing mostly empty math.  Here
// each used expert's packed weight rows are read once per 64 of its routed
// rows, in 16-byte chunks;
// every sum runs in a fixed order, so the result is deterministic.
//
// Kernels (grid over (weight-row block, expert); experts without rows exit):
//   decode_gate_up: a[r] = silu(x[t] Wg_e) * (x[t] Wu_e) for the rows r of
//                   expert e (t = perm[r] / k), from the packed gate/up rows
//                   [E][2I][H] (64-row blocks: 32 gate rows, then the 32 up
//                   rows of the same intermediate indices);
//   decode_down:    y[r] = a[r] Wd_e from the packed down rows [E][H][I].
// The combine that follows is the layer's own (combine_kernel).
//
// The contraction runs on v_mfma_f32_16x16x32_bf16 as a skinny GEMM: A = 16
// routed rows of the expert (up to four such blocks per pass, each with its
// own accumulator, all fed by the same weight load; rows past the expert's
// end repeat its last row and their results are dropped), B = 16 weight rows
// of the wave.  Lane l
// holds row l % 16 of either operand and contraction values
// [8 (l / 16), 8 (l / 16) + 8) of each 32-wide step -- one 16-byte load per
// operand per step, the same k split in A and B -- and receives outputs
// (row 4 (l / 16) + v, weight row l % 16), v = 0..3.  The matrix core does
// the sums, so no cross-lane reduction is needed and a wave keeps only a few
// dozen registers: several waves per SIMD keep enough weight loads in flight
// to stream HBM.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kDecRowBlocks = 4;                 // 16-row blocks per pass
constexpr int kDecRows = 16 * kDecRowBlocks;     // routed rows of one expert per pass
constexpr int kDecBlock = 64;  // weight rows per workgroup (4 waves x 16)
constexpr int kDecUnroll = 4;  // 32-wide steps whose loads are issued together

// acc[p] (16 rows x 16 weight rows) = sum over the K/32 steps of the A rows of
// block p times the wave's weight rows, for the nb (uniform) blocks in use:
// each weight chunk loaded feeds nb MFMAs.  xrow[p]: this lane's A row in
// block p (its 16-byte chunks); wrow: this lane's weight row.
__device__ __forceinline__ void dec_mfma(const uint4 *const *xrow, const uint4 *__restrict__ wrow,
                                         int KC, int nb, f32x4v (&acc)[kDecRowBlocks]) {
  const int lane = threadIdx.x & 63;
  const int c0 = lane >> 4;  // chunk of 8 within a 32-wide step
#pragma unroll
  for (int p = 0; p < kDecRowBlocks; p++) acc[p] = (f32x4v){0.0f, 0.0f, 0.0f, 0.0f};
  const int steps = KC / 4;
  int st = 0;
  for (; st + kDecUnroll <= steps; st += kDecUnroll) {
    uint4 bv[kDecUnroll], av[kDecUnroll][kDecRowBlocks];
#pragma unroll
    for (int u = 0; u < kDecUnroll; u++) {
      bv[u] = wrow[(st + u) * 4 + c0];
#pragma unroll
      for (int p = 0; p < kDecRowBlocks; p++)
        if (p < nb) av[u][p] = xrow[p][(st + u) * 4 + c0];
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; u++) {
      bf16x8 b;
      __builtin_memcpy(&b, &bv[u], 16);
#pragma unroll
      for (int p = 0; p < kDecRowBlocks; p++) {
        if (p < nb) {
          bf16x8 a;
          __builtin_memcpy(&a, &av[u][p], 16);
          acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[p], 0, 0, 0);
        }
      }
    }
  }
  for (; st < steps; st++) {
    const uint4 bv = wrow[st * 4 + c0];
    bf16x8 b;
    __builtin_memcpy(&b, &bv, 16);
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++) {
      if (p < nb) {
        const uint4 av = xrow[p][st * 4 + c0];
        bf16x8 a;
        __builtin_memcpy(&a, &av, 16);
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[p], 0, 0, 0);
      }
    }
  }
}

// dots[wrow][row] of this wave's 16 weight rows for the pass's rows.
__device__ __forceinline__ void dec_store(const f32x4v (&acc)[kDecRowBlocks], int nb,
                                          float (*dots)[kDecRows]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < kDecRowBlocks; p++)
    if (p < nb)
#pragma unroll
      for (int v = 0; v < 4; v++)
        dots[wave * 16 + (lane & 15)][16 * p + 4 * (lane >> 4) + v] = acc[p][v];
}

// perm == nullptr: row r is token r (the shared expert's dense rows).
__global__ __launch_bounds__(256) void decode_gate_up_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const uint16_t *__restrict__ guT,
    uint16_t *__restrict__ act, int k, int H, int I) {
  __shared__ float dots[kDecBlock][kDecRows];
  const int cb = blockIdx.x, e = blockIdx.y;
  const int rb = offsets[e], re = offsets[e + 1];
  if (rb >= re) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, HC = H / 8;
  const uint4 *wrow = (const uint4 *)(guT + ((size_t)e * 2 * I + (size_t)cb * kDecBlock +
                                             wave * 16 + (lane & 15)) * H);
  for (int r0 = rb; r0 < re; r0 += kDecRows) {
    const int nr = min(kDecRows, re - r0), nb = (nr + 15) / 16;
    const uint4 *xrow[kDecRowBlocks];
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++) {
      const int r = r0 + min(16 * p + (lane & 15), nr - 1);
      xrow[p] = (const uint4 *)x + (size_t)(perm ? perm[r] / k : r) * HC;
    }
    f32x4v acc[kDecRowBlocks];
    dec_mfma(xrow, wrow, HC, nb, acc);
    dec_store(acc, nb, dots);
    __syncthreads();
    // packed rows 0-31 of the block are gate rows, 32-63 the matching up rows
    for (int i = threadIdx.x; i < 32 * nr; i += 256) {
      const int j = i & 31, q = i >> 5;
      const float g = dots[j][q], u = dots[32 + j][q];
      act[(size_t)(r0 + q) * I + cb * 32 + j] = (uint16_t)f32_to_bf16(silu_f(g) * u);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void decode_down_kernel(const uint16_t *__restrict__ act,
                                                          const int32_t *__restrict__ offsets,
                                                          const uint16_t *__restrict__ dT,
                                                          uint16_t *__restrict__ y, int H, int I) {
  __shared__ float dots[kDecBlock][kDecRows];
  const int hb = blockIdx.x, e = blockIdx.y;
  const int rb = offsets[e], re = offsets[e + 1];
  if (rb >= re) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, IC = I / 8;
  const uint4 *wrow = (const uint4 *)(dT + ((size_t)e * H + (size_t)hb * kDecBlock + wave * 16 +
                                            (lane & 15)) * I);
  for (int r0 = rb; r0 < re; r0 += kDecRows) {
    const int nr = min(kDecRows, re - r0), nb = (nr + 15) / 16;
    const uint4 *xrow[kDecRowBlocks];
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++)
      xrow[p] = (const uint4 *)act + (size_t)(r0 + min(16 * p + (lane & 15), nr - 1)) * IC;
    f32x4v acc[kDecRowBlocks];
    dec_mfma(xrow, wrow, IC, nb, acc);
    dec_store(acc, nb, dots);
    __syncthreads();
    for (int i = threadIdx.x; i < kDecBlock * nr; i += 256) {
      const int h = i & (kDecBlock - 1), q = i / kDecBlock;
      y[(size_t)(r0 + q) * H + hb * kDecBlock + h] = (uint16_t)f32_to_bf16(dots[h][q]);
    }
    __syncthreads();
  }
}

// Layout of a small routed set in one workgroup (R <= kDecLayoutMax): the
// same stable counting sort as the layer's three layout kernels -- counts[e],
// offsets = exclusive scan, sorted position of flat row f = offsets[idx[f]] +
// the number of f' < f with the same expert -- with the ranks counted in LDS.
__global__ __launch_bounds__(1024) void decode_layout_kernel(const int32_t *__restrict__ idx,
                                                             int R, int E,
                                                             int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ perm,
                                                             int32_t *__restrict__ inv) {
  __shared__ int32_t e_of[kDecLayoutMax];
  __shared__ int32_t cnt[1024], off[1025];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int f = tid; f < R; f += 1024) {
    // out-of-range expert ids are clamped, as the layer's layout kernels do,
    // so a bad id misroutes a row but never addresses memory outside
    const int e = min(max(idx[f], 0), E - 1);
    e_of[f] = e;
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; e++) { off[e] = acc; acc += cnt[e]; }
    off[E] = acc;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) {
    offsets[e] = off[e];
    if (e < E) counts[e] = cnt[e];
  }
  for (int f = tid; f < R; f += 1024) {
    const int e = e_of[f];
    int rank = 0;
    for (int g = 0; g < f; g++) rank += e_of[g] == e;
    const int r = off[e] + rank;
    perm[r] = f;
    inv[f] = r;
  }
}

void launch_decode_layout(const int32_t *idx, int R, int E, int32_t *counts, int32_t *offsets,
                          int32_t *perm, int32_t *inv, hipStream_t s) {
  hipLaunchKernelGGL(decode_layout_kernel, dim3(1), dim3(1024), 0, s, idx, R, E, counts, offsets,
                     perm, inv);
}

void launch_decode_ffn(const uint16_t *x, const int32_t *perm, const int32_t *offsets, int G,
                       int k, int H, int I, const uint16_t *guT, const uint16_t *dT,
                       uint16_t *act, uint16_t *y, hipStream_t s) {
  if (G <= 0) return;
  hipLaunchKernelGGL(decode_gate_up_kernel, dim3(2 * I / kDecBlock, G), dim3(256), 0, s, x, perm,
                     offsets, guT, act, k, H, I);
  hipLaunchKernelGGL(decode_down_kernel, dim3(H / kDecBlock, G), dim3(256), 0, s, act, offsets,
                     dT, y, H, I);
}

}  // namespace moe
