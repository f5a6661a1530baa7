// Grouped GEMMs on MXFP8 operands for the expert FFN's forward GEMMs and its
// backward data gradients: one tile per workgroup, the tile itself in
// row_tile.h.
#include "gemm_common.h"
#include "row_tile.h"

namespace moe {

template <int EPI, int BFMT>
__global__ __launch_bounds__(NT, 1) void gemm_mx_kernel(GemmArgs p, MxOperands mx) {
  __shared__ __attribute__((aligned(1024))) uint8_t L0[2 * BM * MXK];  // [A | B], even stages
  __shared__ __attribute__((aligned(1024))) uint8_t L1[2 * BM * MXK];  // [A | B], odd stages
  const int MT = p.tile_start[p.G];
  const int nN = p.n_tiles_n;
  const int b = blockIdx.x;
  if (b >= MT * nN) return;
  int mt, nt;
  tile_of_block(b, MT, nN, mt, nt);
  int lo = 0, hi = p.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_start[mid] <= mt) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int rowbase = p.offsets[g];
  mx_tile<EPI, BFMT>(p, mx, g, (mt - p.tile_start[g]) * BM, nt * BN, rowbase,
                     p.offsets[g + 1] - rowbase, L0, L1);
}

template <int BFMT>
static void launch_mx_fmt(const GemmArgs &p, const MxOperands &mx, int epi, const dim3 &gr,
                          hipStream_t s) {
  const dim3 b(NT);
  switch (epi) {
    case EPI_BF16:
      hipLaunchKernelGGL((gemm_mx_kernel<EPI_BF16, BFMT>), gr, b, 0, s, p, mx);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_mx_kernel<EPI_SWIGLU, BFMT>), gr, b, 0, s, p, mx);
      break;
    default:
      hipLaunchKernelGGL((gemm_mx_kernel<EPI_SWIGLU_BWD, BFMT>), gr, b, 0, s, p, mx);
      break;
  }
}

void launch_gemm_rows_mx(const GemmArgs &p0, const MxOperands &mx, int epi, int max_rows,
                         hipStream_t s) {
  GemmArgs p = p0;
  p.stamps = current_stamps();
  p.n_tiles_n = (p.N + BN - 1) / BN;
  const long grid = ((long)max_rows / BM + p.G) * p.n_tiles_n;
  if (grid <= 0) return;
  const dim3 gr((unsigned)grid);
  switch (mx.b_fmt) {
    case kMxE2M1: launch_mx_fmt<kMxE2M1>(p, mx, epi, gr, s); break;
    case kMxE2M3: launch_mx_fmt<kMxE2M3>(p, mx, epi, gr, s); break;
    case kMxE3M2: launch_mx_fmt<kMxE3M2>(p, mx, epi, gr, s); break;
    default: launch_mx_fmt<kMxE4M3>(p, mx, epi, gr, s); break;
  }
}

// ---------------------------------------------------------------------------
// Lower-precision MX copies of the expert weights.  One thread per 32-value
// block of a row: s = clamp(floor(log2 amax) - emax, -127, 127) (an all-zero
// block: -127), each value clamped to the format's maximum at scale 2^s and
// rounded to nearest, ties to even, with gradual underflow below the
// smallest normal 2^emin: with e = max(floor(log2 |v|), emin) the code's
// magnitude bits are 2^m (e - emin) + rint(|v| 2^(m - e)), and the sign bit
// is set exactly when v < 0.  Formats: E2M1 (m 1, emin 0, emax 2, max 6),
// E2M3 (m 3, emin 0, emax 2, max 7.5), E3M2 (m 2, emin -2, emax 4, max 28).

struct LowFmt {
  int m, emin, emax, sign_shift;
  float vmax;
};

__device__ __forceinline__ uint32_t low_encode(float v, const LowFmt &f) {
  const float a = fminf(fabsf(v), f.vmax);
  const int e = a < ldexpf(1.0f, f.emin) ? f.emin : floor_log2(a);
  const uint32_t q = (uint32_t)rintf(ldexpf(a, f.m - e));
  return (((uint32_t)(e - f.emin)) << f.m) + q + (v < 0.0f ? (1u << f.sign_shift) : 0u);
}

__global__ __launch_bounds__(256) void quant_rows_low_kernel(const uint16_t *__restrict__ src,
                                                             int rows, int K,
                                                             uint8_t *__restrict__ q,
                                                             uint8_t *__restrict__ sc, int fmt) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  const int nb = K / 32;
  if (id >= (long)rows * nb) return;
  const int r = (int)(id / nb), blk = (int)(id - (long)r * nb);
  const LowFmt f = fmt == kMxE2M1   ? LowFmt{1, 0, 2, 3, 6.0f}
                   : fmt == kMxE2M3 ? LowFmt{3, 0, 2, 5, 7.5f}
                                    : LowFmt{2, -2, 4, 5, 28.0f};
  float v[32];
  const uint4 *p4 = (const uint4 *)(src + (size_t)r * K + blk * 32);
#pragma unroll
  for (int i = 0; i < 4; i++) unpack8(p4[i], v + 8 * i);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  int s = -127;
  if (amax > 0.0f) s = max(-127, min(127, floor_log2(amax) - f.emax));
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int width = fmt == kMxE2M1 ? 4 : 6;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const unsigned long long c = low_encode(ldexpf(v[i], -s), f);
    const int bit = width * i;
    w[bit >> 5] |= (uint32_t)(c << (bit & 31));
    if ((bit & 31) + width > 32) w[(bit >> 5) + 1] |= (uint32_t)(c >> (32 - (bit & 31)));
  }
  if (fmt == kMxE2M1) {
    *(uint4 *)(q + (size_t)r * (K / 2) + blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint4 *d = (uint4 *)(q + (size_t)r * K + blk * 32);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], 0u, 0u);
  }
  sc[((size_t)(blk >> 2) * rows + r) * 4 + (blk & 3)] = (uint8_t)(s + 127);
}

void launch_quant_rows_mx_low(const uint16_t *src, int rows, int K, uint8_t *q, uint8_t *sc,
                              int fmt, hipStream_t s) {
  const long n = (long)rows * (K / 32);
  if (n <= 0) return;
  hipLaunchKernelGGL(quant_rows_low_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     src, rows, K, q, sc, fmt);
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
// row-wise (conflict-free), writes the block's scale byte and puts its 32
// codes into the column's 128-byte line, staged in LDS; the lines leave as
// 16-byte stores, eight lanes per line, so each store instruction writes
// eight whole lines (storing the 32 codes straight from the converting lane
// split every line into 16-byte pieces from different instructions).
__global__ __launch_bounds__(256) void quant_cols_mx_kernel(
    const uint16_t *__restrict__ src, int C, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ poff, int E, long Rp, uint8_t *__restrict__ q,
    uint8_t *__restrict__ sc) {
  __shared__ uint4 tile[MXK][8];  // 128 rows x 64 bf16
  // column j's 128 codes at byte 144 j: the 16-byte pad puts the 64 lanes'
  // writes of one block (stride 144) on distinct banks
  constexpr int kLine = MXK + 16;
  __shared__ __attribute__((aligned(16))) uint8_t lines[64 * kLine];
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
    // each source row is read once in the whole backward (non-temporal)
    tile[row][c8] = (r < rend && c < C) ? ld_once((const uint4 *)(src + (size_t)r * C + c))
                                        : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  const int blk = tid >> 6, j = tid & 63, c = c0 + j;
  {
    const uint16_t *t16 = (const uint16_t *)tile;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; i++) v[i] = bf16_to_f32(t16[(32 * blk + i) * 64 + j]);
    uint32_t w[8];
    const uint32_t s = mx_block32(v, w, nullptr);
    uint4 *ln = (uint4 *)(lines + j * kLine + 32 * blk);
    ln[0] = make_uint4(w[0], w[1], w[2], w[3]);
    ln[1] = make_uint4(w[4], w[5], w[6], w[7]);
    if (c < C) sc[((size_t)st * C + c) * 4 + blk] = (uint8_t)s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int piece = tid + 256 * i, col = piece >> 3, part = piece & 7;
    if (c0 + col < C)
      *(uint4 *)(q + (size_t)(c0 + col) * Rp + kp + 16 * part) =
          *(const uint4 *)(lines + col * kLine + 16 * part);
  }
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
  p.stamps = current_stamps();
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
