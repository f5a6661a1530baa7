// Grouped GEMMs on MXFP8 operands for the expert FFN's forward GEMMs and its
// backward data gradients: one tile per workgroup, the tile itself in
// row_tile.h.
#include "gemm_common.h"
#include "row_tile.h"

namespace moe {

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_mx_kernel(GemmArgs p, MxOperands mx) {
  __shared__ __attribute__((aligned(1024))) uint8_t L0[2 * BM * MXK];  // [A | B], even stages
  __shared__ __attribute__((aligned(1024))) uint8_t L1[2 * BM * MXK];  // [A | B], odd stages
  const int MT = p.tile_start[p.G];
  const int nN = p.n_tiles_n;
  const int b = blockIdx.x;
  if (b >= MT * nN) return;
  const int mt = b / nN, nt = b - (b / nN) * nN;
  int lo = 0, hi = p.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_start[mid] <= mt) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int rowbase = p.offsets[g];
  mx_tile<EPI>(p, mx, g, (mt - p.tile_start[g]) * BM, nt * BN, rowbase,
               p.offsets[g + 1] - rowbase, L0, L1);
}

void launch_gemm_rows_mx(const GemmArgs &p0, const MxOperands &mx, int epi, int max_rows,
                         hipStream_t s) {
  GemmArgs p = p0;
  p.n_tiles_n = (p.N + BN - 1) / BN;
  const long grid = ((long)max_rows / BM + p.G) * p.n_tiles_n;
  if (grid <= 0) return;
  const dim3 gr((unsigned)grid), b(NT);
  switch (epi) {
    case EPI_BF16: hipLaunchKernelGGL(gemm_mx_kernel<EPI_BF16>, gr, b, 0, s, p, mx); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_mx_kernel<EPI_SWIGLU>, gr, b, 0, s, p, mx); break;
    default: hipLaunchKernelGGL(gemm_mx_kernel<EPI_SWIGLU_BWD>, gr, b, 0, s, p, mx); break;
  }
}

// ---------------------------------------------------------------------------
// MX weight gradients.  The weight-gradient GEMMs contract over each
// expert's routed rows, so their MX operands are quantised down the rows:
// E8M0 blocks of 32 consecutive rows of one column, starting at the expert's
// first row, the last block zero-padded.  Both operands are stored
// transposed, [C][Rp] codes (row c = column c of the source, contraction
// contiguous) with K-blocked scales [Rp/128][C][4], and each expert's row
// segment is padded to a multiple of 128 (one GEMM stage), so that expert e
// owns contraction range [poff[e], poff[e+1]) and the MX row tile runs on
// it unchanged.

// poff[e] = sum over e' < e of the expert row counts rounded up to 128
// (one workgroup of 1024 threads, E <= 1024).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t *__restrict__ offsets,
                                                           int E, int32_t *__restrict__ poff) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  const int n = e < E ? offsets[e + 1] - offsets[e] : 0;
  int v = (n + MXK - 1) / MXK * MXK;
  sc[e] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
    const int add = e >= o ? sc[e - o] : 0;
    __syncthreads();
    v += add;
    sc[e] = v;
    __syncthreads();
  }
  if (e < E) poff[e + 1] = v;
  if (e == 0) poff[0] = 0;
}

// Workgroup = (64 columns, one 128-row stage of the padded row space; a stage
// never straddles two experts).  The stage's rows of the 64 columns (zeros
// past the expert's rows) are loaded with 16-byte row-wise loads into LDS;
// then wave q converts 32-row block q, one column per lane, reading LDS
// row-wise (conflict-free), and writes the block's 32 codes to q[c] and its
// scale byte -- the four waves together fill each column's 128-byte line.
__global__ __launch_bounds__(256) void quant_cols_mx_kernel(
    const uint16_t *__restrict__ src, int C, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ poff, int E, long Rp, uint8_t *__restrict__ q,
    uint8_t *__restrict__ sc) {
  __shared__ uint4 tile[MXK][8];  // 128 rows x 64 bf16
  const int c0 = blockIdx.x * 64;
  const int st = blockIdx.y, kp = st * MXK;
  if (kp >= poff[E]) return;  // uniform over the workgroup
  int lo = 0, hi = E;  // poff[lo] <= kp < poff[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (poff[mid] <= kp) lo = mid; else hi = mid;
  }
  const int r0 = offsets[lo] + (kp - poff[lo]), rend = offsets[lo + 1];
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int chunk = tid + 256 * i, row = chunk >> 3, c8 = chunk & 7;
    const int r = r0 + row, c = c0 + 8 * c8;
    tile[row][c8] = (r < rend && c < C) ? *(const uint4 *)(src + (size_t)r * C + c)
                                        : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  const int blk = tid >> 6, j = tid & 63, c = c0 + j;
  if (c >= C) return;
  const uint16_t *t16 = (const uint16_t *)tile;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; i++) v[i] = bf16_to_f32(t16[(32 * blk + i) * 64 + j]);
  uint32_t w[8];
  const uint32_t s = mx_block32(v, w, nullptr);
  uint4 *dst = (uint4 *)(q + (size_t)c * Rp + kp + 32 * blk);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc[((size_t)st * C + c) * 4 + blk] = (uint8_t)s;
}

// One 256 x 256 tile of expert order[gi]'s weight gradient C_e[M][N] =
// A_e^T B_e over its padded contraction range.
template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_mx_wgrad_kernel(GemmArgs p, MxOperands mx) {
  __shared__ __attribute__((aligned(1024))) uint8_t L0[2 * BM * MXK];
  __shared__ __attribute__((aligned(1024))) uint8_t L1[2 * BM * MXK];
  const int per = p.n_tiles_m * p.n_tiles_n;
  const int gi = blockIdx.x / per;
  const int rem = blockIdx.x - gi * per;
  const int g = p.order ? p.order[gi] : gi;
  const int mt = rem / p.n_tiles_n, nt = rem - mt * p.n_tiles_n;
  const int kp = p.offsets[g], Kp = p.offsets[g + 1] - kp;
  GemmArgs q = p;
  q.A = (const uint16_t *)((const uint8_t *)p.A + kp);
  q.B = (const uint16_t *)((const uint8_t *)p.B + kp);
  q.K = Kp;
  q.G = 1;
  q.sB = 0;
  q.C = (float *)p.C + (size_t)g * p.sC;
  q.C2 = p.C2 ? (void *)((float *)p.C2 + (size_t)g * p.sC) : nullptr;
  MxOperands m = mx;
  m.a_scale = mx.a_scale + (size_t)(kp / MXK) * p.M * 4;
  m.b_scale = mx.b_scale + (size_t)(kp / MXK) * p.N * 4;
  m.a_rows = p.M;
  mx_tile<EPI>(q, m, 0, mt * BM, nt * BN, 0, p.M, L0, L1);
}

void launch_pad_offsets(const int32_t *offsets, int E, int32_t *poff, hipStream_t s) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, s, offsets, E, poff);
}

void launch_quant_cols_mx(const uint16_t *src, int R, int C, const int32_t *offsets,
                          const int32_t *poff, int E, long Rp, uint8_t *q, uint8_t *sc,
                          hipStream_t s) {
  (void)R;
  if (C <= 0 || Rp <= 0) return;
  hipLaunchKernelGGL(quant_cols_mx_kernel, dim3((C + 63) / 64, (unsigned)(Rp / MXK)), dim3(256),
                     0, s, src, C, offsets, poff, E, Rp, q, sc);
}

void launch_gemm_mx_wgrad(const GemmArgs &p0, const MxOperands &mx, int epi, hipStream_t s) {
  GemmArgs p = p0;
  p.n_tiles_m = (p.M + BM - 1) / BM;
  p.n_tiles_n = (p.N + BN - 1) / BN;
  const long grid = (long)p.G * p.n_tiles_m * p.n_tiles_n;
  if (grid <= 0) return;
  const dim3 gr((unsigned)grid), b(NT);
  if (epi == EPI_F32)
    hipLaunchKernelGGL(gemm_mx_wgrad_kernel<EPI_F32>, gr, b, 0, s, p, mx);
  else
    hipLaunchKernelGGL(gemm_mx_wgrad_kernel<EPI_WGRAD_GU>, gr, b, 0, s, p, mx);
}

}  // namespace moe
