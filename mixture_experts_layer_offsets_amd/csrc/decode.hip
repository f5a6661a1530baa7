// Few-token (decode) forward of the expert FFN.
//
// noticiai.com.br ("Cursor abre código do Mixture-of-Kittens ...") mentions a
// separate decode kernel for inference, where each token is handled by its
// own small group of threads.  With a handful of tokens the layer is bound by
// reading the selected experts' weights, not by arithmetic: a 256-row MFMA
// tile would stream the same weights while doing mostly empty math.  Here
// each used expert's packed weight rows are read once per 64 of its routed
// rows; every sum runs in a fixed order, so the result is deterministic.
//
// Kernels (grid over (weight-row group, expert), one wave per workgroup;
// experts without rows exit):
//   decode_gate_up: a[r] = silu(x[t] Wg_e) * (x[t] Wu_e) for the rows r of
//                   expert e (t = perm[r] / k), from the packed gate/up rows
//                   [E][2I][H] (64-row blocks: 32 gate rows, then the 32 up
//                   rows of the same intermediate indices); a wave takes 16
//                   intermediate indices: 16 gate and the 16 matching up rows;
//   decode_down:    y[r] = a[r] Wd_e from the packed down rows [E][H][I]; a
//                   wave takes 32 hidden indices.
// The combine that follows is the layer's own (combine_kernel).
//
// The contraction runs on v_mfma_f32_16x16x32_bf16 as a skinny GEMM: A = 16
// routed rows of the expert (up to four such blocks per pass, each with its
// own accumulator; rows past the expert's end repeat its last row and their
// results are dropped), B = 16 weight rows (two such tiles per wave, each
// A load feeding both).  Lane l holds row l % 16 of either operand and
// contraction values [8 (l / 16), 8 (l / 16) + 8) of each 32-wide step --
// one 16-byte chunk per operand and step, the same split in A and B -- and
// receives outputs (row 4 (l / 16) + v, weight row l % 16), v = 0..3; the
// matrix core does the sums, no cross-lane reduction.
//
// Streaming: the weight chunks go by direct-to-LDS DMA into a ring private
// to the wave, D steps ahead of their use (D x 2 KB in flight per wave), and
// the routed rows' chunks into a register ring of the same depth, issued
// together with the same step's weights: loads complete in issue order
// (vmcnt), so the rows must run as far ahead as the weights or the wait for
// them would drain the weight loads too.  Each lane reads back the LDS chunk
// its own DMA lane wrote, so the wave needs no barrier.  Steps past the end
// still issue (a zero-byte weight load, a row reload of step 0) so every
// wait has a fixed count; their MFMAs are skipped.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kDecRowBlocks = 4;              // 16-row blocks per pass
constexpr int kDecRows = 16 * kDecRowBlocks;  // routed rows of one expert per pass
constexpr int kDecTiles = 2;                  // 16-row weight tiles per wave
constexpr int kDecSlotBytes = kDecTiles * 2 * 1024;  // a 64-wide step of both tiles

constexpr int dec_min(int a, int b) { return a < b ? a : b; }

// Ring depth in 64-wide steps for NB row blocks: at most DMAX slots; a wave
// may have at most 63 memory operations outstanding (vmcnt), and one step
// issues 2 kDecTiles weight DMAs and 2 NB row loads; the row ring takes 8 NB
// registers per step, at most XREGS.
constexpr int dec_depth(int NB, int DMAX, int XREGS) {
  return dec_min(dec_min(DMAX, 63 / (2 * kDecTiles + 2 * NB)), XREGS / (8 * NB));
}
// gate/up: K = H, one wave per 16 intermediate indices (few waves per CU);
// down: K = I, one wave per 32 hidden indices (more waves: a 24 KB ring and
// at most 128 row-ring registers, so six waves fit a CU)
constexpr int kDecSlotsGU = 8, kDecXregsGU = 1024;
constexpr int kDecSlotsDown = 6, kDecXregsDown = 128;

// Ring slot J: an LDS object of its own.  The compiler waits for the DMAs
// into an LDS object before reading it, and it tells objects apart (up to
// eight), so a slot's reads wait for that slot's DMA alone; one array for
// the whole ring would make every read wait for every DMA in flight.
template <int J>
__device__ __forceinline__ uint8_t *dec_slot() {
  __shared__ __attribute__((aligned(1024))) uint8_t slot[kDecSlotBytes];
  return slot;
}

// f(integral_constant<int, I>) for I = B .. E - 1, in order (compile-time
// slot and step indices, which LDS objects and immediate offsets need)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// acc[m][p] (16 rows x 16 weight rows) += the pass's rows of block p times
// weight tile m over the K / 64 steps, taken from step `start` on and
// wrapping (a different start per wave spreads the waves that run at once
// over the DRAM channels: rows 2-14 KB apart would otherwise have every wave
// at the same column, and the same channels, at the same time; the order is
// fixed per wave, so the sums are still deterministic).  xrow[p]: this
// lane's chunk of step 0 in its row of block p; wr: the wave's weight rows;
// wo[m]: this lane's byte offset of step 0 in tile m.  A step is two 32-wide
// MFMA steps: per tile two DMAs (16 rows x 64 bytes each), per row block two
// 16-byte loads.
template <int NB, int DMAX, int XREGS>
__device__ __forceinline__ void dec_stream(const uint4 *const *xrow, __amdgpu_buffer_rsrc_t wr,
                                           const uint32_t *wo, int steps, int start,
                                           f32x4v (&acc)[kDecTiles][kDecRowBlocks]) {
  constexpr int D = dec_depth(NB, DMAX, XREGS);
  constexpr int kOps = 2 * kDecTiles + 2 * NB;  // memory operations per step
  const int lane = threadIdx.x & 63;
  uint4 xv[D][NB][2];
  // The s-th step (uniform) into slot J, the same instructions for every
  // step with no branch (the compiler's waits assume one issue order); past
  // the end: a lane offset beyond the descriptor (zero fill, no traffic) and
  // the row chunks of step 0 (never used).  The DMAs take the step's byte
  // offset as their scalar offset (an immediate offset would also move the
  // LDS destination).
  auto issue = [&](int s, auto J) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    uint8_t *L = dec_slot<j>();
    const int dead = s >= steps;  // uniform
    int se = s + start;
    se = se >= steps ? se - steps : se;
    se = dead ? 0 : se;
    const uint32_t far = (0u - (uint32_t)dead) & 0x7FFFF000u;
    const uint32_t so = (uint32_t)se * 128u;
#pragma unroll
    for (int m = 0; m < kDecTiles; m++) {
      const uint32_t vo = wo[m] | far;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(L + 2 * m * 1024), 16, vo, so, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(L + (2 * m + 1) * 1024), 16, vo,
                                               so + 64, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < NB; p++) {
      const uint4 *q = xrow[p] + se * 8;
      xv[j][p][0] = q[0];
      xv[j][p][1] = q[4];
    }
  };
  // The prologue in the loop's issue order (each step's DMAs, then its row
  // loads): the compiler's waits for the row registers at the loop head
  // assume that order.  The empty asm with a memory clobber keeps every
  // pass from moving the row loads across it (they touch no LDS, so the
  // DMAs would not hold them); it emits nothing and adds no wait.
  static_for<0, D>([&](auto J) __attribute__((always_inline)) {
    issue(J, J);
    asm volatile("" ::: "memory");
  });
  for (int s0 = 0; s0 < steps; s0 += D) {
    static_for<0, D>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      // step s0 + j has landed when only the D - 1 later steps are pending
      __builtin_amdgcn_s_waitcnt(vmcnt_wait((D - 1) * kOps));
      if (s0 + j < steps) {
        const uint8_t *L = dec_slot<j>();
        bf16x8 b[kDecTiles][2];
#pragma unroll
        for (int m = 0; m < kDecTiles; m++)
#pragma unroll
          for (int i = 0; i < 2; i++)
            __builtin_memcpy(&b[m][i], L + (2 * m + i) * 1024 + lane * 16, 16);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int p = 0; p < NB; p++) {
            bf16x8 a;
            __builtin_memcpy(&a, &xv[j][p][i], 16);
#pragma unroll
            for (int m = 0; m < kDecTiles; m++)
              acc[m][p] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[m][i], acc[m][p], 0, 0, 0);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      // after the slot's reads (their MFMAs used them)
      issue(s0 + j + D, J);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);  // no DMA into the ring outlives the pass
}

// One pass over up to kDecRows rows of the expert: nb (uniform) row blocks.
template <int DMAX, int XREGS>
__device__ __forceinline__ void dec_pass(int nb, const uint4 *const *xrow,
                                         __amdgpu_buffer_rsrc_t wr, const uint32_t *wo, int steps,
                                         int start, f32x4v (&acc)[kDecTiles][kDecRowBlocks]) {
#pragma unroll
  for (int m = 0; m < kDecTiles; m++)
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++) acc[m][p] = (f32x4v){0.0f, 0.0f, 0.0f, 0.0f};
  switch (nb) {
    case 1: dec_stream<1, DMAX, XREGS>(xrow, wr, wo, steps, start, acc); break;
    case 2: dec_stream<2, DMAX, XREGS>(xrow, wr, wo, steps, start, acc); break;
    case 3: dec_stream<3, DMAX, XREGS>(xrow, wr, wo, steps, start, acc); break;
    default: dec_stream<4, DMAX, XREGS>(xrow, wr, wo, steps, start, acc); break;
  }
}

// perm == nullptr: row r is token r (the shared expert's dense rows).  The
// row operands (x here, act in decode_down) are deliberately not
// __restrict__: loads through a restrict-qualified read-only argument are
// taken out of the memory ordering, and then no barrier keeps them in the
// ring's issue order.
__global__ __launch_bounds__(64) void decode_gate_up_kernel(
    const uint16_t *x, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const uint16_t *__restrict__ guT,
    uint16_t *__restrict__ act, int k, int H, int I) {
  const int i0 = blockIdx.x * 16, e = blockIdx.y;
  const int rb = offsets[e], re = offsets[e + 1];
  if (rb >= re) return;
  const int lane = threadIdx.x, HC = H / 8;
  const int start = (blockIdx.x + 5 * blockIdx.y) % (H / 64);  // this wave's first step
  // gate rows i0 .. i0 + 15 sit at packed row 64 (i0 / 32) + i0 % 32, the
  // matching up rows 32 packed rows further
  const uint16_t *w0 = guT + ((size_t)e * 2 * I + (size_t)(i0 / 32) * 64 + i0 % 32) * H;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void *)w0, (short)0, 48 * H * 2, kBufferDword3);
  uint32_t wo[kDecTiles];
#pragma unroll
  for (int m = 0; m < kDecTiles; m++)
    wo[m] = (uint32_t)((32 * m + (lane & 15)) * H * 2 + (lane >> 4) * 16);
  for (int r0 = rb + blockIdx.z * kDecRows; r0 < re; r0 += gridDim.z * kDecRows) {
    const int nr = min(kDecRows, re - r0), nb = (nr + 15) / 16;
    const uint4 *xrow[kDecRowBlocks];
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++) {
      const int r = r0 + min(16 * p + (lane & 15), nr - 1);
      xrow[p] = (const uint4 *)x + (size_t)(perm ? perm[r] / k : r) * HC + (lane >> 4);
    }
    f32x4v acc[kDecTiles][kDecRowBlocks];
    dec_pass<kDecSlotsGU, kDecXregsGU>(nb, xrow, wr, wo, H / 64, start, acc);
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int q = 16 * p + 4 * (lane >> 4) + v;
        if (p < nb && q < nr)
          act[(size_t)(r0 + q) * I + i0 + (lane & 15)] =
              (uint16_t)f32_to_bf16(silu_f(acc[0][p][v]) * acc[1][p][v]);
      }
  }
}

__global__ __launch_bounds__(64) void decode_down_kernel(const uint16_t *act,
                                                         const int32_t *__restrict__ offsets,
                                                         const uint16_t *__restrict__ dT,
                                                         uint16_t *__restrict__ y, int H, int I) {
  const int h0 = blockIdx.x * 32, e = blockIdx.y;
  const int rb = offsets[e], re = offsets[e + 1];
  if (rb >= re) return;
  const int lane = threadIdx.x, IC = I / 8;
  const int start = (blockIdx.x + 5 * blockIdx.y) % (I / 64);  // this wave's first step
  const uint16_t *w0 = dT + ((size_t)e * H + h0) * I;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void *)w0, (short)0, 32 * I * 2, kBufferDword3);
  uint32_t wo[kDecTiles];
#pragma unroll
  for (int m = 0; m < kDecTiles; m++)
    wo[m] = (uint32_t)((16 * m + (lane & 15)) * I * 2 + (lane >> 4) * 16);
  for (int r0 = rb + blockIdx.z * kDecRows; r0 < re; r0 += gridDim.z * kDecRows) {
    const int nr = min(kDecRows, re - r0), nb = (nr + 15) / 16;
    const uint4 *xrow[kDecRowBlocks];
#pragma unroll
    for (int p = 0; p < kDecRowBlocks; p++)
      xrow[p] = (const uint4 *)act + (size_t)(r0 + min(16 * p + (lane & 15), nr - 1)) * IC +
                (lane >> 4);
    f32x4v acc[kDecTiles][kDecRowBlocks];
    dec_pass<kDecSlotsDown, kDecXregsDown>(nb, xrow, wr, wo, I / 64, start, acc);
#pragma unroll
    for (int m = 0; m < kDecTiles; m++)
#pragma unroll
      for (int p = 0; p < kDecRowBlocks; p++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          const int q = 16 * p + 4 * (lane >> 4) + v;
          if (p < nb && q < nr)
            y[(size_t)(r0 + q) * H + h0 + 16 * m + (lane & 15)] =
                (uint16_t)f32_to_bf16(acc[m][p][v]);
        }
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
                       long rows, int k, int H, int I, const uint16_t *guT, const uint16_t *dT,
                       uint16_t *act, uint16_t *y, hipStream_t s) {
  if (G <= 0 || rows <= 0) return;
  // one wave per 16 intermediate indices (gate/up) or 32 hidden indices
  // (down) and per 64-row pass (grid z: enough passes for a group holding all
  // `rows`; a wave past its group's last pass exits at once), so the passes
  // of a group with many rows run side by side instead of one after another
  // in the same waves; H and I are multiples of 64
  const unsigned passes = (unsigned)std::min<long>((rows + kDecRows - 1) / kDecRows, 65535);
  hipLaunchKernelGGL(decode_gate_up_kernel, dim3(I / 16, G, passes), dim3(64), 0, s, x, perm,
                     offsets, guT, act, k, H, I);
  hipLaunchKernelGGL(decode_down_kernel, dim3(H / 32, G, passes), dim3(64), 0, s, act, offsets,
                     dT, y, H, I);
}

}  // namespace moe
