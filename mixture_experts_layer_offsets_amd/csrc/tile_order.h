// Workgroup -> tile orders of the expert GEMMs.  Workgroups go to the eight
// XCDs of the device in turn (workgroup b to XCD b mod 8), and each XCD has
// an L2 of its own, so the order decides which XCD reads which operand
// panels.  Plain integer functions, compiled for the device by the kernels
// and for the host by tests/tile_order_check.cpp.
#pragma once

#if defined(__HIPCC__)
#define TILE_ORDER_FN __host__ __device__ __forceinline__
#else
#define TILE_ORDER_FN inline
#endif

namespace moe {

TILE_ORDER_FN int tile_order_min(int a, int b) { return a < b ? a : b; }

// Tile of a row-ragged GEMM for workgroup b (MT row tiles x nN column tiles,
// b < MT nN).  Each XCD runs 32 of every 256 consecutive workgroups at once;
// the remap hands those 32 a compact block of 4 row tiles x 8 column tiles,
// taken from bands of 8 column tiles (row tiles fastest across blocks), so a
// row panel is read by one XCD's L2 instead of by all eight.  Full rounds of
// 256 are permuted; a last partial round keeps the band order.  Measured on
// MI355X: up to 5 % faster for 8 column tiles (with the plain n-fastest order
// each XCD then holds one column and 32 row panels), neutral for 16 and 28.
TILE_ORDER_FN void tile_of_block(int b, int MT, int nN, int &mt, int &nt) {
  const int total = MT * nN, full = total & ~255;
  const int k = b < full ? ((((b >> 8) << 3) + (b & 7)) << 5) + ((b & 255) >> 3) : b;
  const int nb = (nN + 7) >> 3, per = MT << 3;
  const int beta = tile_order_min(k / per, nb - 1), kk = k - beta * per;
  const int w = tile_order_min(8, nN - (beta << 3));
  mt = kk / w;
  nt = (beta << 3) + kk - (kk / w) * w;
}

// Group index gi (into the processing order) and tile index rem (row-major
// over the group's `per` tiles) of weight-gradient workgroup b, over G groups
// of `per` tiles each.  Plain order: group by group.  XCD-major order (G a
// multiple of 8): XCD x takes all tiles of groups x, x + 8, ..., so each
// group's operand rows are read by one XCD, whose concurrent tiles share them
// in its L2; in the plain order a tile's column index picks its XCD and
// every XCD fetches every group's A panel.
TILE_ORDER_FN void wgrad_tile_of_block(int b, int per, bool xcd_major, int &gi, int &rem) {
  if (xcd_major) {
    const int x = b & 7, j = b >> 3, q = j / per;
    gi = q * 8 + x;
    rem = j - q * per;
  } else {
    gi = b / per;
    rem = b - gi * per;
  }
}

}  // namespace moe
