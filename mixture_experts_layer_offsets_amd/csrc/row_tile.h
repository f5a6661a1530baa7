// One 256 x 256 output tile of a row-ragged grouped GEMM, as device
// functions: the one-tile-per-workgroup kernels and the persistent layer
// kernel both call them.
#pragma once

#include "gemm_common.h"
#include "mx_device.h"
#include "tile_epilogue.h"

namespace moe {

// Row-ragged GEMM with both operands contraction-contiguous (the forward
// gate/up and down GEMMs and both backward data-gradient GEMMs).
//
// Operands move from HBM straight into LDS with buffer_load_dwordx4 ... lds:
// no staging registers and no ds_write instructions.  A wave's 16-byte load
// lands lane-linearly in a 1 KB LDS segment (8 rows of 128 bytes), so each
// lane fetches the global chunk that the XOR swizzle assigns to its LDS slot.
// The buffer descriptor covers exactly the tile's valid rows: rows past the
// end of the group read as zeros, with no per-row masks.  Two LDS buffers
// (separate arrays, so the compiler can tell the one being filled from the
// one being read) alternate per 64-deep K slice; MFMA fragments are double
// buffered in registers so LDS latency hides behind the previous 16 MFMAs.
//
// The tile covers rows [rowbase + m0, rowbase + min(m0 + 256, Mg)) of A and
// the B matrix of group g; L0, L1 are the workgroup's two 64 KB LDS buffers.
template <int EPI>
__device__ __forceinline__ void nt_tile(const GemmArgs &p, int g, int m0, int n0, int rowbase,
                                        int Mg, uint16_t *L0, uint16_t *L1) {
  TileClock clk;
  clk.start(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;
  const int a_rows = min(BM, Mg - m0), b_rows = min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(p.A + (size_t)(rowbase + m0) * p.lda), (short)0, a_rows * (int)p.lda * 2,
      kBufferDword3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(p.B + (size_t)g * p.sB + (size_t)n0 * p.ldb), (short)0, b_rows * (int)p.ldb * 2,
      kBufferDword3);
  uint32_t oa[8], ob[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swz5(row);
    oa[i] = (uint32_t)(row * (int)p.lda * 2 + kc * 16);
    ob[i] = (uint32_t)(row * (int)p.ldb * 2 + kc * 16);
  }
  // A stage index past the end selects empty descriptors: the DMA then writes
  // zeros into the (no longer read) buffer and touches no memory.  This keeps
  // the K loop free of branches, across which the compiler could otherwise
  // sink a k-slice's MFMAs past the barrier.
  const __amdgpu_buffer_rsrc_t rNone =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, 0, kBufferDword3);
  // DMA instruction q (0-7: A rows, 8-15: B rows) of stage kt into L.
  auto dma = [&](uint16_t *L, int kt, int q) {
    const bool live = kt < p.K / BK;
    const int soff = live ? kt * BK * 2 : 0;
    if (q < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rA : rNone,
                                               (lds_ptr_t)(L + (wave * 8 + q) * 512), 16, oa[q],
                                               soff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          live ? rB : rNone, (lds_ptr_t)(L + BM * BK + (wave * 8 + q - 8) * 512), 16, ob[q - 8],
          soff, 0, 0);
  };
  auto issue = [&](uint16_t *L, int kt) {
#pragma unroll
    for (int q = 0; q < 16; q++) dma(L, kt, q);
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (f32x16){};
  const int fr = lane & 31;
  const int cA = swz5(fr) ^ (lane >> 5);
  const int baseA = (wm0 + fr) * BK, baseB = BM * BK + (wn0 + fr) * BK;
  int offk[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++) offk[ks] = ((2 * ks) ^ cA) << 3;
  // Fragments double-buffered across the whole K loop: in each stage, the
  // wait for the next stage's operands and the barrier come after the third
  // k-slice's MFMAs are issued (they keep the matrix pipe busy meanwhile),
  // and the next stage's first fragments load while the last slice's MFMAs
  // run.  Set s & 1 holds the fragments of k-slice s of a stage.
  bf16x8 fa[2][4], fb[2][4];
  auto load = [&](const uint16_t *L, int ks, int set) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      fa[set][i] = *(const bf16x8 *)(L + baseA + i * 32 * BK + offk[ks]);
      fb[set][i] = *(const bf16x8 *)(L + baseB + i * 32 * BK + offk[ks]);
    }
  };
  auto mma = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0,
                                                            0, 0);
  };
  const int nk = p.K / BK;
  // Lc holds stage kt, Ln receives stage kt + 1 (in flight); Lc is refilled
  // with stage kt + 2 once every wave has its last fragments of stage kt.
  // The refill's 16 DMA instructions are spread over 32 MFMAs: 0-7 after
  // every second MFMA of the last k-slice, 8-15 after every second MFMA of
  // the next stage's first slice.  Issued as one burst they stall the wave
  // whenever the memory pipeline is backed up, and no MFMA issues meanwhile.
  auto mma_dma = [&](int set, uint16_t *Ld, int dkt, int d0) {
#pragma unroll
    for (int q = 0; q < 16; q++) {
      acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          fa[set][q >> 2], fb[set][q & 3], acc[q >> 2][q & 3], 0, 0, 0);
      if (q & 1) dma(Ld, dkt, d0 + (q >> 1));  // zeros past the end
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // `first`: stage 0, whose successor the prologue issued in full
  auto stage = [&](uint16_t *Lc, uint16_t *Ln, int kt, auto first) {
    load(Lc, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(first)::value)
      mma(0);
    else
      mma_dma(0, Ln, kt + 1, 8);  // second half of Ln's refill
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
    mma_dma(1, Lc, kt + 2, 0);  // first half of Lc's refill
  };
  // Prologue: stages 0 and 1 in flight together, then the wait for stage 0
  // alone (its 16 DMAs were issued first): one memory latency per tile.
  issue(L0, 0);
  issue(L1, 1);
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
  __syncthreads();                      // the epilogue reuses both buffers
  clk.loop_done(p);
  const TileAt t{m0, n0, rowbase, Mg, wm0, wn0, lane, tid};
  if constexpr (EPI == EPI_BF16)
    tile_epi_bf16(p, acc, (uint8_t *)L0, (uint8_t *)L1, t);
  else if constexpr (EPI == EPI_SWIGLU)
    tile_epi_swiglu<false>(p, nullptr, acc, (uint8_t *)L0, (uint8_t *)L1, t);
  else
    tile_epi_swiglu_bwd(p, acc, (uint8_t *)L0, (uint8_t *)L1, t);
  clk.finish(p);
}

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
// The SwiGLU epilogue can quantise a = silu(g) * u along I (see
// tile_epilogue.h).
constexpr int MXK = 128;  // K bytes (= fp8 values) per stage

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Lower-precision B operands (the expert weights of the lower-precision
// variants; A stays E4M3).  Measured on MI355X for the f8f6f4 instruction
// with an FP4 or FP6 B operand: lane l supplies column l & 31, and lane half
// h the 32 consecutive K values of block h, packed little-endian (value p at
// bits [W p, W p + W), W = 4 or 6): 16 bytes per block for FP4, 24 for FP6.
// FP4 rows are stored packed (64 bytes per 128-value stage, four 16-byte
// chunks, swizzled within the row by swz4); FP6 blocks sit in 32-byte slots
// (24 bytes of codes, 8 of zeros) so an FP6 row has the FP8 row's geometry.
// BFMT is the instruction's B format code: 0 E4M3, 2 FP6 E2M3, 3 FP6 E3M2,
// 4 FP4 E2M1.
__device__ __forceinline__ int swz4(int row) { return (row ^ (row >> 2)) & 3; }

// The MX tile; same geometry and buffers as nt_tile.
template <int EPI, int BFMT = kMxE4M3>
__device__ __forceinline__ void mx_tile(const GemmArgs &p, const MxOperands &mx, int g, int m0,
                                        int n0, int rowbase, int Mg, uint8_t *L0, uint8_t *L1) {
  TileClock clk;
  clk.start(p);
  // B bytes per row and stage, and B DMA instructions per wave and stage
  constexpr int BKB = BFMT == kMxE2M1 ? MXK / 2 : MXK;
  constexpr int NBQ = BFMT == kMxE2M1 ? 4 : 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;
  const int a_rows = min(BM, Mg - m0), b_rows = min(BN, p.N - n0);
  const int K = p.K, KS = K / 32;  // bytes per row of codes / of scales

  const uint8_t *Ac = (const uint8_t *)p.A, *Bc = (const uint8_t *)p.B;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Ac + (size_t)(rowbase + m0) * p.lda), (short)0, a_rows * (int)p.lda, kBufferDword3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Bc + (size_t)g * p.sB + (size_t)n0 * p.ldb), (short)0, b_rows * (int)p.ldb,
      kBufferDword3);
  // K-blocked scales: stage kt's dword for A row r at (kt * a_rows + r) * 4,
  // for B row n of group g at (kt * G*N + g*N + n) * 4
  const int b_rows_all = p.G * p.N;
  const __amdgpu_buffer_rsrc_t rSa = __builtin_amdgcn_make_buffer_rsrc(
      (void *)mx.a_scale, (short)0, mx.a_rows * KS, kBufferDword3);
  const __amdgpu_buffer_rsrc_t rSb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)mx.b_scale, (short)0, b_rows_all * KS, kBufferDword3);
  const int sa_row = rowbase + m0 + wm0, sb_row = g * p.N + n0 + wn0;

  uint32_t oa[8], ob[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swz5(row);
    oa[i] = (uint32_t)(row * (int)p.lda + kc * 16);
    if constexpr (BFMT == kMxE2M1) {
      // 16 rows of four 16-byte chunks per instruction
      const int rb = (wave * 4 + (i & 3)) * 16 + (lane >> 2);
      ob[i] = (uint32_t)(rb * (int)p.ldb + (((lane & 3) ^ swz4(rb)) * 16));
    } else {
      ob[i] = (uint32_t)(row * (int)p.ldb + kc * 16);
    }
  }
  // A stage index past the end selects empty descriptors: the DMA then writes
  // zeros into the (no longer read) buffer and touches no memory.  This keeps
  // the main loop free of branches, which would let the compiler sink the
  // MFMAs of a k-slice past the barrier and collapse the pipeline.
  const __amdgpu_buffer_rsrc_t rNone =
      __builtin_amdgcn_make_buffer_rsrc((void *)Ac, (short)0, 0, kBufferDword3);
  // DMA instruction q (0-7: A rows, 8 .. 8+NBQ-1: B rows) of stage kt into L.
  auto dma = [&](uint8_t *L, int kt, int q) {
    const bool live = kt < K / MXK;
    const int soff = live ? kt * MXK : 0;
    if (q < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rA : rNone,
                                               (lds_ptr_t)(L + (wave * 8 + q) * 1024), 16, oa[q],
                                               soff, 0, 0);
    else if (q < 8 + NBQ)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          live ? rB : rNone, (lds_ptr_t)(L + BM * MXK + (wave * NBQ + q - 8) * 1024), 16,
          ob[q - 8], BKB == MXK ? soff : soff / 2, 0, 0);
  };
  auto issue = [&](uint8_t *L, int kt) {
#pragma unroll
    for (int q = 0; q < 8 + NBQ; q++) dma(L, kt, q);
  };
  // scale dwords of this lane's rows (4 blocks of 32 along K per stage); 32
  // consecutive rows' dwords are one 128-byte line
  const int fr = lane & 31, h = lane >> 5;
  auto load_scales = [&](int kt, int *sa, int *sb) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sa[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rSa, (kt * mx.a_rows + sa_row + 32 * i + fr) * 4, 0, 0);
      sb[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rSb, (kt * b_rows_all + sb_row + 32 * i + fr) * 4, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (f32x16){};

  const int sw = swz5(fr);
  const int baseA = (wm0 + fr) * MXK, baseB = BM * MXK + (wn0 + fr) * BKB;
  // Same pipeline as nt_tile, with two 64-deep k-slices per stage: slice 1's
  // fragments load while slice 0's MFMAs run, then the wait and the barrier,
  // then the next stage's slice-0 fragments load while slice 1's MFMAs run.
  // Scale dwords for stage kt + 2 are fetched after slice 1's MFMAs are
  // issued (they reuse stage kt's registers) and arrive by the next wait.
  i32x8 fa[2][4], fb[2][4];
  auto load = [&](const uint8_t *L, int ks, int set) {
    const int c0 = ((4 * ks + h) ^ sw) << 4, c1 = ((4 * ks + 2 + h) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 x0 = *(const uint4 *)(L + baseA + i * 32 * MXK + c0);
      const uint4 x1 = *(const uint4 *)(L + baseA + i * 32 * MXK + c1);
      fa[set][i] = (i32x8){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                           (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      if constexpr (BFMT == kMxE4M3) {
        const uint4 y0 = *(const uint4 *)(L + baseB + i * 32 * BKB + c0);
        const uint4 y1 = *(const uint4 *)(L + baseB + i * 32 * BKB + c1);
        fb[set][i] = (i32x8){(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w,
                             (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
      } else if constexpr (BFMT == kMxE2M1) {
        // block 2ks + h: one 16-byte chunk
        const uint4 y0 =
            *(const uint4 *)(L + baseB + i * 32 * BKB + (((2 * ks + h) ^ swz4(fr)) << 4));
        fb[set][i] = (i32x8){(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, 0, 0, 0, 0};
      } else {
        // block 2ks + h: the 32-byte slot's two chunks (24 bytes of codes)
        const int b2 = 2 * (2 * ks + h);
        const uint4 y0 = *(const uint4 *)(L + baseB + i * 32 * BKB + ((b2 ^ sw) << 4));
        const uint4 y1 = *(const uint4 *)(L + baseB + i * 32 * BKB + (((b2 + 1) ^ sw) << 4));
        fb[set][i] = (i32x8){(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w,
                             (int)y1.x, (int)y1.y, 0, 0};
      }
    }
  };
  auto mma1 = [&](int ks, int i, int j, const int *sa, const int *sb) {
    const int sh = 8 * (2 * ks + h);
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fa[ks][i], fb[ks][j], acc[i][j], 0, BFMT, 0, (sa[i] >> sh) & 0xFF, 0,
        (sb[j] >> sh) & 0xFF);
  };
  auto mma = [&](int ks, const int *sa, const int *sb) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) mma1(ks, i, j, sa, sb);
  };

  const int nk = K / MXK;
  int sa0[4], sb0[4], sa1[4], sb1[4];
  // Lc holds stage kt (scales sa, sb), Ln receives stage kt + 1.
  auto stage = [&](uint8_t *Lc, const uint8_t *Ln, int kt, int *sa, int *sb) {
    load(Lc, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(0, sa, sb);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    load(Ln, 0, 0);  // after the last stage this reads zeros, unused
    __builtin_amdgcn_sched_barrier(0);
    // the refill's DMA instructions one after each MFMA (see nt_tile)
#pragma unroll
    for (int q = 0; q < 16; q++) {
      mma1(1, q >> 2, q & 3, sa, sb);
      dma(Lc, kt + 2, q);  // zeros past the end
      __builtin_amdgcn_sched_barrier(0);
    }
    load_scales(min(kt + 2, nk - 1), sa, sb);
  };
  // Prologue: stages 0 and 1 (and their scales) in flight together, then
  // the wait for stage 0 and its scales alone (stage 1's 8 + NBQ DMAs and 8
  // scale loads were issued after them): one memory latency per tile.  The
  // empty asm with a memory clobber keeps that order: without it the
  // scheduler issued all 16 + 2 NBQ DMAs before the scale loads, the wait
  // no longer covered stage 0's scales, and the compiler's own waits for
  // them at the loop head then held every second stage until the DMAs
  // issued during the stage before it had landed.
  issue(L0, 0);
  load_scales(0, sa0, sb0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  issue(L1, 1);
  load_scales(min(1, nk - 1), sa1, sb1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(8 + NBQ + 8));
  barrier_after_wait();
  load(L0, 0, 0);
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    stage(L0, L1, kt, sa0, sb0);
    stage(L1, L0, kt + 1, sa1, sb1);
  }
  if (kt < nk) stage(L0, L1, kt, sa0, sb0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);  // the zero fills
  __syncthreads();  // the epilogue reuses both buffers
  clk.loop_done(p);

  const TileAt t{m0, n0, rowbase, Mg, wm0, wn0, lane, tid};
  if constexpr (EPI == EPI_BF16) {
    tile_epi_bf16(p, acc, L0, L1, t);
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (mx.q_out)
      tile_epi_swiglu<true>(p, &mx, acc, L0, L1, t);
    else
      tile_epi_swiglu<false>(p, nullptr, acc, L0, L1, t);
  } else if constexpr (EPI == EPI_F32 || EPI == EPI_WGRAD_GU) {
    // weight gradients (fp32, p.C / p.C2 already at the group's matrix)
    epilogue<true, EPI>(p, acc, 0, m0, n0, 0, Mg, wm0, wn0, lane);
  } else {
    tile_epi_swiglu_bwd(p, acc, L0, L1, t);
  }
  clk.finish(p);
}

}  // namespace moe
