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
  int mt, nt;
  tile_of_block(b, MT, nN, mt, nt);
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

// ---------------------------------------------------------------------------
// Weight-gradient GEMM with both operands row-major over the contraction:
// C_g[M][N] = sum over the group's rows r of A[r][M]^T B[r][N].
//
// The 64-row K slices of A and B (rows of 256 M or N values, 512 bytes) move
// into LDS untransposed by direct-to-LDS DMA, exactly as they lie in HBM; the
// buffer descriptor starts at the group's first row and ends at its last, so
// the ragged K tail reads zeros.  The MFMA fragments (8 consecutive k of one
// m per lane) are then read with ds_read_b64_tr_b16, gfx950's transposing LDS
// read: within each 16-lane group, output lane 4a + b receives element b of
// the 4-element chunks addressed by lanes a, 4 + a, 8 + a and 12 + a
// (measured on MI355X).  Lane j of a group therefore addresses row
// k0 + j/4 at column base + 4 (j % 4), and two such reads (k0, k0 + 4) give
// a lane its 8 k values.  16-byte chunks are XOR-swizzled by 4 (k & 3) so the
// four rows one read touches land in four different bank groups.

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 *lds_v4i16_t;

__device__ __forceinline__ int tn_swz(int k) { return (k & 3) << 2; }

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_tn_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t L0[2 * 64 * BM];  // [A | B], even stages
  __shared__ __attribute__((aligned(1024))) uint16_t L1[2 * 64 * BM];  // [A | B], odd stages
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;
  const int per = p.n_tiles_m * p.n_tiles_n;
  int gi, rem;  // plain or XCD-major order (tile_order.h, launch_gemm_wgrad)
  wgrad_tile_of_block(blockIdx.x, per, p.xcd_major != 0, gi, rem);
  const int g = p.order ? p.order[gi] : gi;
  const int mt = rem / p.n_tiles_n;
  const int m0 = mt * BM, n0 = (rem - mt * p.n_tiles_n) * BN;
  const int koff = p.offsets[g];
  const int Kg = p.offsets[g + 1] - koff;
  TileClock clk;
  clk.start(p);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (f32x16){};

  if (Kg > 0) {
    const uint16_t *gA = p.A + (size_t)koff * p.lda + m0;  // the group's first row,
    const uint16_t *gB = p.B + (size_t)koff * p.ldb + n0;  // from the tile's column
    // DMA: instruction i of wave w fills LDS rows 2 (8w + i) + {0, 1}; lane L
    // writes chunk L % 32 of row 2 (8w + i) + L / 32 and so fetches the global
    // chunk that the swizzle maps there.
    uint32_t oa[8], ob[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = 2 * (wave * 8 + i) + (lane >> 5);
      const int c = (lane & 31) ^ tn_swz(row);
      oa[i] = (uint32_t)(row * (int)p.lda * 2 + c * 16);
      ob[i] = (uint32_t)(row * (int)p.ldb * 2 + c * 16);
    }
    const int nk = (Kg + 63) / 64;
    // The descriptor of stage kt's A (B) rows starts at the stage's first
    // row, so its byte count and offsets stay within 64 rows however long
    // the group; it ends at column M (N) of the group's last row, so rows
    // past the group and a partial column tile read zeros, nothing outside
    // the operands; a stage past the end gets zero bytes (zero fill, no
    // traffic).  Built once per stage and operand: built per instruction, or
    // selected between descriptors, it cost branches and private memory.
    auto desc = [&](int kt, bool a) {
      const int rows = Kg - kt * 64;
      const int ld = a ? (int)p.lda : (int)p.ldb;
      const int bytes =
          rows <= 0 ? 0 : ((min(rows, 64) - 1) * ld + (a ? p.M - m0 : p.N - n0)) * 2;
      return __builtin_amdgcn_make_buffer_rsrc((void *)((a ? gA : gB) + (size_t)kt * 64 * ld),
                                               (short)0, bytes, kBufferDword3);
    };
    // DMA instruction q (0-7: A rows, 8-15: B rows) of a stage into L
    auto dma = [&](__amdgpu_buffer_rsrc_t r, uint16_t *L, int q) {
      if (q < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(L + (wave * 8 + q) * 512), 16,
                                                 oa[q], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_ptr_t)(L + 64 * BM + (wave * 8 + q - 8) * 512), 16, ob[q - 8], 0, 0, 0);
    };
    // fragment addresses: lane l in 16-lane group q = l / 16, j = l % 16
    const int q = lane >> 4, j = lane & 15;
    const int krow = 8 * (q >> 1) + (j >> 2);          // + 16 ks + {0, 4}
    const int colA = wm0 + 16 * (q & 1) + 4 * (j & 3);  // + 32 i
    const int colB = wn0 + 16 * (q & 1) + 4 * (j & 3);  // + 32 i
    // element offset of (row k, column c) in an operand slice
    auto off = [](int k, int c) { return k * BM + (((c >> 3) ^ tn_swz(k)) << 3) + (c & 7); };
    auto frag = [&](const uint16_t *T, int k0, int c) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(T + off(k0, c)));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(T + off(k0 + 4, c)));
      bf16x8 f;
      const v4i16 *plo = &lo, *phi = &hi;
      __builtin_memcpy(&f, plo, 8);
      __builtin_memcpy((char *)&f + 8, phi, 8);
      return f;
    };
    // The row-ragged tile's pipeline (row_tile.h): fragments double buffered
    // across the whole K loop; the wait and the barrier after the third
    // k-slice; the refill of the buffer just finished (stage kt + 2) spread
    // over 32 MFMAs, DMAs 0-7 after every second MFMA of the last slice and
    // 8-15 after every second MFMA of the next stage's first slice.
    bf16x8 fa[2][4], fb[2][4];
    auto load = [&](const uint16_t *L, int ks, int set) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        fa[set][i] = frag(L, 16 * ks + krow, colA + 32 * i);
        fb[set][i] = frag(L + 64 * BM, 16 * ks + krow, colB + 32 * i);
      }
    };
    auto mma = [&](int set) {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][jj],
                                                               acc[i][jj], 0, 0, 0);
    };
    // 16 MFMAs with DMAs d0 .. d0 + 7 of stage dkt (descriptor r) between
    auto mma_dma = [&](int set, uint16_t *Ld, __amdgpu_buffer_rsrc_t r, int d0) {
#pragma unroll
      for (int q = 0; q < 16; q++) {
        acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            fa[set][q >> 2], fb[set][q & 3], acc[q >> 2][q & 3], 0, 0, 0);
        if (q & 1) dma(r, Ld, d0 + (q >> 1));  // zeros past the end
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // `first`: stage 0, whose successor the prologue issued in full
    auto stage = [&](uint16_t *Lc, uint16_t *Ln, int kt, auto first) {
      const __amdgpu_buffer_rsrc_t rb = desc(kt + 1, false), ra = desc(kt + 2, true);
      load(Lc, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(first)::value)
        mma(0);
      else
        mma_dma(0, Ln, rb, 8);  // second half of Ln's refill
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 1; ks < 3; ks++) {
        load(Lc, ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(ks & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      load(Ln, 0, 0);  // after the last stage this reads zeros, unused
      __builtin_amdgcn_sched_barrier(0);
      mma_dma(1, Lc, ra, 0);  // first half of Lc's refill
    };
    // Prologue: stages 0 and 1 in flight together, then the wait for stage 0
    // alone (its 16 DMAs were issued first), so a short contraction (a few
    // stages: experts with few rows) pays one memory latency up front, not
    // two.
    {
      const __amdgpu_buffer_rsrc_t a0 = desc(0, true), b0 = desc(0, false);
      const __amdgpu_buffer_rsrc_t a1 = desc(1, true), b1 = desc(1, false);
#pragma unroll
      for (int q = 0; q < 16; q++) dma(q < 8 ? a0 : b0, L0, q);
#pragma unroll
      for (int q = 0; q < 16; q++) dma(q < 8 ? a1 : b1, L1, q);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(16));
    barrier_after_wait();
    load(L0, 0, 0);
    stage(L0, L1, 0, std::true_type{});
    int kt = 1;
    for (; kt + 2 <= nk; kt += 2) {
      stage(L1, L0, kt, std::false_type{});
      stage(L0, L1, kt + 1, std::false_type{});
    }
    if (kt < nk) stage(L1, L0, kt, std::false_type{});
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // the zero fills
  }
  clk.loop_done(p);
  epilogue<true, EPI>(p, acc, g, m0, n0, 0, p.M, wm0, wn0, lane);
  clk.finish(p);
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
  p.stamps = current_stamps();
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

void launch_gemm_wgrad(const GemmArgs &p0, int epi, long rows, hipStream_t s) {
  GemmArgs p = p0;
  p.stamps = current_stamps();
  p.n_tiles_m = (p.M + BM - 1) / BM;
  p.n_tiles_n = (p.N + BN - 1) / BN;
  const long grid = (long)p.G * p.n_tiles_m * p.n_tiles_n;
  if (grid <= 0) return;
  // XCD-major tile order when the groups are many (a multiple of 8, so every
  // XCD gets as many) and an average group's operand rows, rows / G x (M + N)
  // bf16 values, fit one XCD's 4 MB L2, so that each XCD reads them once.
  // Measured: the 64-expert mid layer's weight gradients 4-6 % faster; with
  // the DeepSeek-V3 share's larger groups (4.7 and 5.8 MB) the down one was
  // 2 % faster and the gate/up one 8 % slower.
  p.xcd_major = p.G % 8 == 0 && p.G >= 16 && rows / p.G * (long)(p.M + p.N) * 2 <= (4L << 20);
  if (p.lda % 8 == 0 && p.ldb % 8 == 0 && p.lda >= BM && p.ldb >= BN &&
      (epi == EPI_F32 || epi == EPI_WGRAD_GU)) {
    const dim3 gr((unsigned)grid), b(NT);
    if (epi == EPI_F32)
      hipLaunchKernelGGL(gemm_tn_kernel<EPI_F32>, gr, b, 0, s, p);
    else
      hipLaunchKernelGGL(gemm_tn_kernel<EPI_WGRAD_GU>, gr, b, 0, s, p);
    return;
  }
  launch_epi<true, false>(p, epi, (int)grid, s);
}

}  // namespace moe
