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

}  // namespace moe
