// Grouped GEMMs on MXFP8 operands (E4M3 codes with one E8M0 scale per 32
// values along K) for the expert FFN's forward GEMMs and its backward data
// gradients.  The pages fuse MXFP8 activation quantisation into the dispatch,
// grouped-GEMM and SwiGLU data paths (kucoin.com news flash "O MoK do Cursor
// alcança aumento de desempenho de 2,37x no NVIDIA GB300 NVL72", §02;
// deepdigest.ru article on MoK).
//
// Same tile and operand feed as the bf16 kernel: 256 x 256 outputs per
// 256-thread workgroup, four waves of 128 x 128, operands DMA'd into LDS in
// 128-byte-deep stages (128 fp8 values per row), double buffered.  The matrix
// instruction is v_mfma_scale_f32_32x32x64_f8f6f4: for a row (or column) of
// the 32 x 64 operand, lane half h holds K bytes [16h, 16h+16) and
// [32+16h, 32+16h+16), and the scale byte it supplies applies to the 32-wide
// K block h (measured on MI355X).  Each fragment is therefore two 16-byte LDS
// reads, and each lane reads one scale dword per 32-row block per stage.
//
// The SwiGLU epilogue can quantise a = silu(g) * u along I on the fly: the 32
// columns of one I-block sit in the 32 lanes of a half-wave, so the block
// maximum is a five-step xor-shuffle reduction.
#include "gemm_common.h"
#include "mx_device.h"
#include "tile_epilogue.h"

namespace moe {

constexpr int MXK = 128;  // K bytes (= fp8 values) per stage

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_mx_kernel(GemmArgs p, MxOperands mx) {
  __shared__ __attribute__((aligned(1024))) uint8_t L0[2 * BM * MXK];  // [A | B], even stages
  __shared__ __attribute__((aligned(1024))) uint8_t L1[2 * BM * MXK];  // [A | B], odd stages
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;

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
  const int m0 = (mt - p.tile_start[g]) * BM;
  const int n0 = nt * BN;
  const int rowbase = p.offsets[g];
  const int Mg = p.offsets[g + 1] - rowbase;
  const int a_rows = min(BM, Mg - m0), b_rows = min(BN, p.N - n0);
  const int K = p.K, KS = K / 32;  // bytes per row of codes / of scales

  const uint8_t *Ac = (const uint8_t *)p.A, *Bc = (const uint8_t *)p.B;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Ac + (size_t)(rowbase + m0) * p.lda), (short)0, a_rows * (int)p.lda, kBufferDword3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Bc + (size_t)g * p.sB + (size_t)n0 * p.ldb), (short)0, b_rows * (int)p.ldb,
      kBufferDword3);
  const __amdgpu_buffer_rsrc_t rSa = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(mx.a_scale + (size_t)(rowbase + m0) * KS), (short)0, a_rows * KS, kBufferDword3);
  const __amdgpu_buffer_rsrc_t rSb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(mx.b_scale + (size_t)g * mx.sBs + (size_t)n0 * KS), (short)0, b_rows * KS,
      kBufferDword3);

  uint32_t oa[8], ob[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swz5(row);
    oa[i] = (uint32_t)(row * (int)p.lda + kc * 16);
    ob[i] = (uint32_t)(row * (int)p.ldb + kc * 16);
  }
  auto issue = [&](uint8_t *L, int kt) {
    const int soff = kt * MXK;
#pragma unroll
    for (int i = 0; i < 8; i++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(L + (wave * 8 + i) * 1024), 16,
                                               oa[i], soff, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; i++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(L + BM * MXK + (wave * 8 + i) * 1024),
                                               16, ob[i], soff, 0, 0);
  };
  // scale dwords of this lane's rows: 4 blocks of 32 along K per stage
  const int fr = lane & 31, h = lane >> 5;
  auto load_scales = [&](int kt, int *sa, int *sb) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sa[i] = __builtin_amdgcn_raw_buffer_load_b32(rSa, (wm0 + 32 * i + fr) * KS + kt * 4, 0, 0);
      sb[i] = __builtin_amdgcn_raw_buffer_load_b32(rSb, (wn0 + 32 * i + fr) * KS + kt * 4, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (f32x16){};

  const int sw = swz5(fr);
  const int baseA = (wm0 + fr) * MXK, baseB = BM * MXK + (wn0 + fr) * MXK;
  auto compute = [&](const uint8_t *L, const int *sa, const int *sb) {
    i32x8 fa[2][4], fb[2][4];
    auto load = [&](int ks, int set) {
      const int c0 = ((4 * ks + h) ^ sw) << 4, c1 = ((4 * ks + 2 + h) ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 x0 = *(const uint4 *)(L + baseA + i * 32 * MXK + c0);
        const uint4 x1 = *(const uint4 *)(L + baseA + i * 32 * MXK + c1);
        fa[set][i] = (i32x8){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                             (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        const uint4 y0 = *(const uint4 *)(L + baseB + i * 32 * MXK + c0);
        const uint4 y1 = *(const uint4 *)(L + baseB + i * 32 * MXK + c1);
        fb[set][i] = (i32x8){(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w,
                             (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
      }
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      if (ks == 0) load(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      const int sh = 8 * (2 * ks + h);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0, (sa[i] >> sh) & 0xFF, 0,
              (sb[j] >> sh) & 0xFF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = K / MXK;
  int sa0[4], sb0[4], sa1[4], sb1[4];
  issue(L0, 0);
  load_scales(0, sa0, sb0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    issue(L1, kt + 1);
    load_scales(kt + 1, sa1, sb1);
    __builtin_amdgcn_sched_barrier(0);
    compute(L0, sa0, sb0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 2 < nk) {
      issue(L0, kt + 2);
      load_scales(kt + 2, sa0, sb0);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(L1, sa1, sb1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (kt < nk) compute(L0, sa0, sb0);

  const TileAt t{m0, n0, rowbase, Mg, wm0, wn0, lane, tid};
  if constexpr (EPI == EPI_BF16) {
    tile_epi_bf16(p, acc, L0, L1, t);
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (mx.q_out)
      tile_epi_swiglu<true>(p, &mx, acc, L0, L1, t);
    else
      tile_epi_swiglu<false>(p, nullptr, acc, L0, L1, t);
  } else {
    tile_epi_swiglu_bwd(p, acc, L0, L1, t);
  }
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
