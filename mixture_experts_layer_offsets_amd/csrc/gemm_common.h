// Tile geometry, LDS swizzles and the epilogue shared by the grouped GEMMs.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tile_order.h"

namespace moe {

constexpr int BM = kTileM, BN = kTileN, BK = kTileK, NT = 256;

__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * BK + ((kc ^ ((row ^ (row >> 3)) & 7)) << 3);
}

// 8x8 transpose of bf16: in[i] holds 8 values along the contiguous axis for
// contraction index i; out[j] holds the 8 contraction values of column j.
__device__ __forceinline__ void transpose8x8(const uint4 *in, uint4 *out) {
  uint32_t a[8][4];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i][0] = in[i].x; a[i][1] = in[i].y; a[i][2] = in[i].z; a[i][3] = in[i].w;
  }
#pragma unroll
  for (int j = 0; j < 8; j++) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint32_t lo = a[2 * q][j >> 1], hi = a[2 * q + 1][j >> 1];
      d[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    out[j] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// 4 x 4 transpose of fp32 values across the four lanes of a quad: lane s of
// the quad holds x[0..3], rows 0..3 of its column s; afterwards it holds row
// s of columns 0..3.  Two butterfly stages of DPP quad permutations (swap
// with lane ^ 1, then with lane ^ 2), each lane sending the value its
// partner keeps.
__device__ __forceinline__ void quad_transpose4(float (&x)[4], int s) {
  const bool odd = s & 1, hi = s & 2;
  auto swap1 = [](float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  };
  auto swap2 = [](float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  };
  const float r0 = swap1(odd ? x[0] : x[1]), r1 = swap1(odd ? x[2] : x[3]);
  const float y0 = odd ? r0 : x[0], y1 = odd ? x[1] : r0;
  const float y2 = odd ? r1 : x[2], y3 = odd ? x[3] : r1;
  const float t0 = swap2(hi ? y0 : y2), t1 = swap2(hi ? y1 : y3);
  x[0] = hi ? t0 : y0;
  x[1] = hi ? t1 : y1;
  x[2] = hi ? y2 : t0;
  x[3] = hi ? y3 : t1;
}

// Epilogue shared by both kernels.  acc[i][j][v] holds row
// wm0 + 32i + 8(v/4) + 4(lane/32) + v%4 and column wn0 + 32j + lane%32 of the tile.
// Weight-gradient fp32 outputs: each 4-row run of the four columns a lane
// quad holds is transposed across the quad (quad_transpose4), so a lane
// writes 4 consecutive columns of one row with one 16-byte store, and a
// wave's store covers eight whole 128-byte lines.  The stores are
// non-temporal: the gradients are not read again here, and with many
// experts of few rows (every tile a short contraction and 256 KB of fp32)
// they otherwise crowd the operands out of the caches (measured on MI355X:
// 8 % faster on the DeepSeek-V3-shaped weight gradients).
template <bool WGRAD, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &p, f32x16 (&acc)[4][4], int g, int m0,
                                         int n0, int rowbase, int Mg, int wm0, int wn0,
                                         int lane) {
  const int N = p.N;
  const int ncol = lane & 31;
  if constexpr (WGRAD && (EPI == EPI_F32 || EPI == EPI_WGRAD_GU)) {
    const int s = lane & 3, c4 = ncol & ~3;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int vq = 0; vq < 4; vq++) {
          float x[4] = {acc[i][j][4 * vq], acc[i][j][4 * vq + 1], acc[i][j][4 * vq + 2],
                        acc[i][j][4 * vq + 3]};
          quad_transpose4(x, s);
          const int m = m0 + wm0 + 32 * i + 8 * vq + 4 * (lane >> 5) + s;
          const int n = n0 + wn0 + 32 * j + c4;
          if (m < Mg && n < N) {
            if constexpr (EPI == EPI_F32) {
              float4 v = make_float4(x[0], x[1], x[2], x[3]);
              if (p.bias) {
                v.x += p.bias[n]; v.y += p.bias[n + 1]; v.z += p.bias[n + 2]; v.w += p.bias[n + 3];
              }
              st_once((uint4 *)((float *)p.C + (size_t)g * p.sC + (size_t)m * p.ldc + n),
                      make_uint4(__float_as_uint(v.x), __float_as_uint(v.y),
                                 __float_as_uint(v.z), __float_as_uint(v.w)));
            } else {
              // packed columns -> dW_gate / dW_up [g][h][i]
              const int ii = (n >> 6) * 32 + (n & 31);
              float *D = (float *)(((n >> 5) & 1) ? p.C2 : p.C) + (size_t)g * p.sC;
              st_once((uint4 *)(D + (size_t)m * p.ldc + ii),
                      make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                                 __float_as_uint(x[2]), __float_as_uint(x[3])));
            }
          }
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int m = m0 + wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (m >= Mg) continue;
      if constexpr (EPI == EPI_BF16) {
        uint16_t *C = (uint16_t *)p.C + (size_t)(rowbase + m) * p.ldc;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int n = n0 + wn0 + j * 32 + ncol;
          if (n < N) C[n] = (uint16_t)f32_to_bf16(acc[i][j][v]);
        }
      } else if constexpr (EPI == EPI_F32) {
        float *C = WGRAD ? (float *)p.C + (size_t)g * p.sC + (size_t)m * p.ldc
                         : (float *)p.C + (size_t)(rowbase + m) * p.ldc;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int n = n0 + wn0 + j * 32 + ncol;
          if (n < N) C[n] = acc[i][j][v] + (p.bias ? p.bias[n] : 0.0f);
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
        // packed columns: 64-column blocks of [32 gate | 32 up]
        uint16_t *A = (uint16_t *)p.C + (size_t)(rowbase + m) * p.ldc;
        uint16_t *GU = p.C2 ? (uint16_t *)p.C2 + (size_t)(rowbase + m) * p.ldc2 : nullptr;
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
          const int n = n0 + wn0 + jj * 64 + ncol;  // gate column
          if (n < N) {
            const float gv = acc[i][2 * jj][v], uv = acc[i][2 * jj + 1][v];
            A[(n >> 6) * 32 + ncol] = (uint16_t)f32_to_bf16(silu_f(gv) * uv);
            if (GU) {
              GU[n] = (uint16_t)f32_to_bf16(gv);
              GU[n + 32] = (uint16_t)f32_to_bf16(uv);
            }
          }
        }
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        // columns are intermediate indices i; read g, u; write dg, du packed
        const uint16_t *GU = p.aux + (size_t)(rowbase + m) * p.ldaux;
        uint16_t *DH = (uint16_t *)p.C + (size_t)(rowbase + m) * p.ldc;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int n = n0 + wn0 + j * 32 + ncol;
          if (n < N) {
            const int pg = (n >> 5) * 64 + (n & 31);
            const float gv = bf16_to_f32(GU[pg]), uv = bf16_to_f32(GU[pg + 32]);
            const float dA = acc[i][j][v];
            const float s = sigmoid_f(gv);
            DH[pg] = (uint16_t)f32_to_bf16(dA * uv * s * (1.0f + gv * (1.0f - s)));
            DH[pg + 32] = (uint16_t)f32_to_bf16(dA * gv * s);
          }
        }
      } else if constexpr (EPI == EPI_WGRAD_GU) {
        // rows h, packed columns -> dW_gate / dW_up [g][h][i]
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int n = n0 + wn0 + j * 32 + ncol;
          if (n < N) {
            const int ii = (n >> 6) * 32 + (n & 31);
            float *D = (float *)(((n >> 5) & 1) ? p.C2 : p.C) + (size_t)g * p.sC;
            D[(size_t)m * p.ldc + ii] = acc[i][j][v];
          }
        }
      }
    }
  }
}

// In-kernel timing of one tile (kernels.h, kStamp*): read only when the
// launch carries a counter block, added by thread 0 with vector atomics.
struct TileClock {
  unsigned long long c0 = 0, r0 = 0, c1 = 0;
  __device__ __forceinline__ void start(const GemmArgs &p) {
    if (p.stamps) {
      c0 = __builtin_amdgcn_s_memtime();
      r0 = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ __forceinline__ void loop_done(const GemmArgs &p) {
    if (p.stamps) c1 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void finish(const GemmArgs &p) {
    if (p.stamps && threadIdx.x == 0) {
      const unsigned long long c2 = __builtin_amdgcn_s_memtime();
      const unsigned long long r2 = __builtin_amdgcn_s_memrealtime();
      atomicAdd(p.stamps + kStampTiles, 1ull);
      atomicAdd(p.stamps + kStampCycles, c2 - c0);
      atomicAdd(p.stamps + kStampLoop, c1 - c0);
      atomicAdd(p.stamps + kStampEpilogue, c2 - c1);
      atomicAdd(p.stamps + kStampTicks, r2 - r0);
    }
  }
};

constexpr uint32_t kBufferDword3 = 0x00020000;  // raw buffer, gfx9 family

// s_waitcnt vmcnt(0) with the other counters left alone, issued through the
// builtin: the compiler's own wait insertion sees it (inline asm it does not)
// and so knows that every vector-memory load issued before it has arrived.
constexpr int kVmcnt0 = 0x0F70;
// s_waitcnt vmcnt(n), 0 <= n < 64 (vmcnt bits [3:0] and [15:14]): all but
// the wave's last n vector-memory loads have arrived (loads count down in
// issue order).
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert(vmcnt_wait(0) == kVmcnt0, "s_waitcnt encoding");

// Workgroup barrier without a memory fence.  __syncthreads' release fence
// makes the compiler wait for every outstanding LDS DMA (vmcnt(0)), also the
// next stage's, which a prologue leaves in flight on purpose; the caller
// waits (s_waitcnt) for the DMAs the barrier must cover, so that after it
// every wave's share of them is in LDS.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_after_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left alone (vmcnt field 63,
// expcnt 7): this wave's LDS reads and writes have completed.
constexpr int kLgkmcnt0 = 0xC07F;

// Workgroup barrier for LDS data written with ds_write: every wave's LDS
// accesses before it have completed, its DMAs and stores may still be in
// flight (no fence, see barrier_after_wait).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Chunk swizzle of the DMA-fed tiles (rows of 64 bf16 = eight 16-byte
// chunks).  It uses row bits 0..4 only: the rows read by any 8 (or 16)
// consecutive lanes of an MFMA fragment land in distinct bank groups, and the
// fragment addresses of the four 32-row blocks differ by immediates only.
__device__ __forceinline__ int swz5(int row) { return (row & 7) ^ ((row >> 3) & 3); }

}  // namespace moe
