// Tile geometry, LDS swizzles and the epilogue shared by the grouped GEMMs.
#pragma once

#include "common.h"
#include "kernels.h"

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

// Epilogue shared by both kernels.  acc[i][j][v] holds row
// wm0 + 32i + 8(v/4) + 4(lane/32) + v%4 and column wn0 + 32j + lane%32 of the tile.
template <bool WGRAD, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &p, f32x16 (&acc)[4][4], int g, int m0,
                                         int n0, int rowbase, int Mg, int wm0, int wn0,
                                         int lane) {
  const int N = p.N;
  const int ncol = lane & 31;
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

// Tile of a row-ragged GEMM for workgroup b (MT row tiles x nN column tiles,
// b < MT nN).  Workgroups go to the eight XCDs in turn (b mod 8), so each
// XCD runs 32 of every 256 consecutive workgroups at once; the remap hands
// those 32 a compact block of 4 row tiles x 8 column tiles, taken from bands
// of 8 column tiles (row tiles fastest across blocks), so a row panel is
// read by one XCD's L2 instead of by all eight.  Full rounds of 256 are
// permuted; a last partial round keeps the band order.  Measured on MI355X:
// up to 5 % faster for 8 column tiles (with the plain n-fastest order each
// XCD then holds one column and 32 row panels), neutral for 16 and 28.
__device__ __forceinline__ void tile_of_block(int b, int MT, int nN, int &mt, int &nt) {
  const int total = MT * nN, full = total & ~255;
  const int k = b < full ? ((((b >> 8) << 3) + (b & 7)) << 5) + ((b & 255) >> 3) : b;
  const int nb = (nN + 7) >> 3, per = MT << 3;
  const int beta = min(k / per, nb - 1), kk = k - beta * per, w = min(8, nN - (beta << 3));
  mt = kk / w;
  nt = (beta << 3) + kk - (kk / w) * w;
}

constexpr uint32_t kBufferDword3 = 0x00020000;  // raw buffer, gfx9 family

// s_waitcnt vmcnt(0) with the other counters left alone, issued through the
// builtin: the compiler's own wait insertion sees it (inline asm it does not)
// and so knows that every vector-memory load issued before it has arrived.
constexpr int kVmcnt0 = 0x0F70;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Chunk swizzle of the DMA-fed tiles (rows of 64 bf16 = eight 16-byte
// chunks).  It uses row bits 0..4 only: the rows read by any 8 (or 16)
// consecutive lanes of an MFMA fragment land in distinct bank groups, and the
// fragment addresses of the four 32-row blocks differ by immediates only.
__device__ __forceinline__ int swz5(int row) { return (row & 7) ^ ((row >> 3) & 3); }

}  // namespace moe
