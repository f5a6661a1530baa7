// Grouped GEMMs of the expert FFN on CDNA4 matrix cores.
//
// The pages' expert FFN is a grouped GEMM over expert-contiguous rows that
// feeds the tensor cores (kucoin.com news flash "O MoK do Cursor alcança
// aumento de desempenho de 2,37x no NVIDIA GB300 NVL72", §01), with SwiGLU in
// its data path (§02).  Here one kernel template serves every GEMM of the
// layer's forward and backward:
//
//   row-ragged mode (forward gate/up and down, backward data gradients):
//     group g owns rows [offsets[g], offsets[g+1]); its tiles are enumerated
//     on the device from a tile prefix, so no host readback sizes the grid.
//   weight-gradient mode: group g's output is a fixed M x N matrix and the
//     contraction runs over the group's rows (a ragged K); groups are visited
//     heaviest first so the long tiles start early.
//
// Tile: 256 x 256 outputs per 256-thread workgroup, four waves of 128 x 128,
// each wave a 4 x 4 grid of v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs).
// Operands are staged through LDS in 64-deep K slices, double buffered.
//   * gemm_nt_kernel (both operands contraction-contiguous: the forward
//     GEMMs and the backward data gradients) moves operands with
//     buffer_load_dwordx4 ... lds straight into an XOR-swizzled LDS layout.
//   * grouped_gemm_kernel (weight gradients and the router, where an operand
//     is contiguous along M or N) loads 8x8 blocks into registers and
//     transposes them on the way into the same LDS layout.
// Measured on MI355X: the MFMA ceiling of this instruction with one wave per
// SIMD is ~2.1 PFLOP/s, and a CU's L2->LDS feed tops out near 34 B/clk --
// about what a 256 x 256 bf16 tile consumes at full MFMA rate -- so the
// kernels are co-limited by operand feed and matrix issue.
#include "gemm_common.h"
#include "row_tile.h"

namespace moe {

template <bool WGRAD, bool B_KC, int EPI>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;

  // ---- which tile
  int g, m0, n0, rowbase, Mg, Kg, koff;
  {
    const int tile = blockIdx.x;
    if constexpr (!WGRAD) {
      const int mt = tile / p.n_tiles_n;
      const int nt = tile - mt * p.n_tiles_n;
      if (mt >= p.tile_start[p.G]) return;
      int lo = 0, hi = p.G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.tile_start[mid] <= mt) lo = mid; else hi = mid;
      }
      g = lo;
      m0 = (mt - p.tile_start[g]) * BM;
      n0 = nt * BN;
      rowbase = p.offsets[g];
      Mg = p.offsets[g + 1] - rowbase;
      Kg = p.K;
      koff = 0;
    } else {
      const int per = p.n_tiles_m * p.n_tiles_n;
      const int gi = tile / per;
      const int rem = tile - gi * per;
      g = p.order ? p.order[gi] : gi;
      const int mt = rem / p.n_tiles_n;
      m0 = mt * BM;
      n0 = (rem - mt * p.n_tiles_n) * BN;
      rowbase = 0;
      Mg = p.M;
      koff = p.offsets[g];
      Kg = p.offsets[g + 1] - koff;
    }
  }
  const int N = p.N;

  // ---- global -> register staging
  uint4 ra[8], rb[8];
  auto load_a = [&](int k0) {
    if constexpr (!WGRAD) {  // A [rows][K], K contiguous
      const int kc = tid & 7;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int row = (tid >> 3) + 32 * i;
        ra[i] = (m0 + row < Mg)
                    ? *(const uint4 *)(p.A + (size_t)(rowbase + m0 + row) * p.lda + k0 + kc * 8)
                    : make_uint4(0, 0, 0, 0);
      }
    } else {  // A [rows = K][M], M contiguous
      const int mc = tid & 31, kg = tid >> 5;
      const bool mok = m0 + mc * 8 < Mg;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int k = k0 + kg * 8 + i;
        ra[i] = (mok && k < Kg)
                    ? *(const uint4 *)(p.A + (size_t)(koff + k) * p.lda + m0 + mc * 8)
                    : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto load_b = [&](int k0) {
    if constexpr (B_KC) {  // B_g [N][K], K contiguous
      const uint16_t *Bg = p.B + (size_t)g * p.sB;
      const int kc = tid & 7;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int row = (tid >> 3) + 32 * i;
        rb[i] = (n0 + row < N) ? *(const uint4 *)(Bg + (size_t)(n0 + row) * p.ldb + k0 + kc * 8)
                               : make_uint4(0, 0, 0, 0);
      }
    } else {  // B [K rows][N], N contiguous (rows offset by the group in wgrad mode)
      const uint16_t *Bg = WGRAD ? p.B : p.B + (size_t)g * p.sB;
      const int nc = tid & 31, kg = tid >> 5;
      const bool nok = n0 + nc * 8 < N;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int k = k0 + kg * 8 + i;
        rb[i] = (nok && k < Kg) ? *(const uint4 *)(Bg + (size_t)(koff + k) * p.ldb + n0 + nc * 8)
                                : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_a = [&](int buf) {
    if constexpr (!WGRAD) {
      const int kc = tid & 7;
#pragma unroll
      for (int i = 0; i < 8; i++)
        *(uint4 *)&sA[buf][lds_off((tid >> 3) + 32 * i, kc)] = ra[i];
    } else {
      uint4 o[8];
      transpose8x8(ra, o);
      const int mc = tid & 31, kg = tid >> 5;
#pragma unroll
      for (int j = 0; j < 8; j++) *(uint4 *)&sA[buf][lds_off(mc * 8 + j, kg)] = o[j];
    }
  };
  auto store_b = [&](int buf) {
    if constexpr (B_KC) {
      const int kc = tid & 7;
#pragma unroll
      for (int i = 0; i < 8; i++)
        *(uint4 *)&sB[buf][lds_off((tid >> 3) + 32 * i, kc)] = rb[i];
    } else {
      uint4 o[8];
      transpose8x8(rb, o);
      const int nc = tid & 31, kg = tid >> 5;
#pragma unroll
      for (int j = 0; j < 8; j++) *(uint4 *)&sB[buf][lds_off(nc * 8 + j, kg)] = o[j];
    }
  };

  // ---- main loop
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (f32x16){};

  const int nk = (Kg + BK - 1) / BK;
  if (nk > 0) {
    load_a(0);
    load_b(0);
    store_a(0);
    store_b(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_a((kt + 1) * BK);
      load_b((kt + 1) * BK);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      const int kc = ks * 2 + (lane >> 5);
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        fa[i] = *(const bf16x8 *)&sA[cur][lds_off(wm0 + i * 32 + (lane & 31), kc)];
#pragma unroll
      for (int j = 0; j < 4; j++)
        fb[j] = *(const bf16x8 *)&sB[cur][lds_off(wn0 + j * 32 + (lane & 31), kc)];
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_a(cur ^ 1);
      store_b(cur ^ 1);
    }
    __syncthreads();
  }

  epilogue<WGRAD, EPI>(p, acc, g, m0, n0, rowbase, Mg, wm0, wn0, lane);
}

// ---------------------------------------------------------------------------
// Row-ragged GEMM with both operands contraction-contiguous (the forward
// gate/up and down GEMMs and both backward data-gradient GEMMs); one tile per
// workgroup, the tile itself in row_tile.h.

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_nt_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t L0[2 * BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t L1[2 * BM * BK];
  const int MT = p.tile_start[p.G];
  const int nN = p.n_tiles_n;
  const int b = blockIdx.x;
  if (b >= MT * nN) return;
  // consecutive blocks share the A row tile (n fastest); measured faster on
  // this chip than XCD-grouped rasters for these shapes
  const int mt = b / nN, nt = b - (b / nN) * nN;
  int lo = 0, hi = p.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_start[mid] <= mt) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int rowbase = p.offsets[g];
  nt_tile<EPI>(p, g, (mt - p.tile_start[g]) * BM, nt * BN, rowbase, p.offsets[g + 1] - rowbase,
               L0, L1);
}

template <bool WGRAD, bool B_KC>
static void launch_epi(const GemmArgs &p, int epi, int grid, hipStream_t s) {
  const dim3 g(grid), b(NT);
  switch (epi) {
    case EPI_BF16: hipLaunchKernelGGL((grouped_gemm_kernel<WGRAD, B_KC, EPI_BF16>), g, b, 0, s, p); break;
    case EPI_F32: hipLaunchKernelGGL((grouped_gemm_kernel<WGRAD, B_KC, EPI_F32>), g, b, 0, s, p); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((grouped_gemm_kernel<WGRAD, B_KC, EPI_SWIGLU>), g, b, 0, s, p); break;
    case EPI_SWIGLU_BWD: hipLaunchKernelGGL((grouped_gemm_kernel<WGRAD, B_KC, EPI_SWIGLU_BWD>), g, b, 0, s, p); break;
    case EPI_WGRAD_GU: hipLaunchKernelGGL((grouped_gemm_kernel<WGRAD, B_KC, EPI_WGRAD_GU>), g, b, 0, s, p); break;
  }
}

void launch_gemm_rows(const GemmArgs &p0, int epi, bool b_kcontig, int max_rows, hipStream_t s) {
  GemmArgs p = p0;
  p.n_tiles_n = (p.N + BN - 1) / BN;
  const long m_tiles = (long)max_rows / BM + p.G;
  const long grid = m_tiles * p.n_tiles_n;
  if (grid <= 0) return;
  if (b_kcontig && p.K % BK == 0 &&
      (epi == EPI_BF16 || epi == EPI_SWIGLU || epi == EPI_SWIGLU_BWD)) {
    const dim3 gr((unsigned)grid), b(NT);
    switch (epi) {
      case EPI_BF16: hipLaunchKernelGGL(gemm_nt_kernel<EPI_BF16>, gr, b, 0, s, p); break;
      case EPI_SWIGLU: hipLaunchKernelGGL(gemm_nt_kernel<EPI_SWIGLU>, gr, b, 0, s, p); break;
      default: hipLaunchKernelGGL(gemm_nt_kernel<EPI_SWIGLU_BWD>, gr, b, 0, s, p); break;
    }
    return;
  }
  if (b_kcontig) launch_epi<false, true>(p, epi, (int)grid, s);
  else launch_epi<false, false>(p, epi, (int)grid, s);
}

void launch_gemm_wgrad(const GemmArgs &p0, int epi, hipStream_t s) {
  GemmArgs p = p0;
  p.n_tiles_m = (p.M + BM - 1) / BM;
  p.n_tiles_n = (p.N + BN - 1) / BN;
  const long grid = (long)p.G * p.n_tiles_m * p.n_tiles_n;
  if (grid <= 0) return;
  launch_epi<true, false>(p, epi, (int)grid, s);
}

}  // namespace moe
