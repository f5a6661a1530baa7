// Row-GEMM epilogues that stage the 256 x 256 output tile in LDS and write
// it out as whole rows with 16-byte stores.
//
// An MFMA accumulator lane holds one column of 4-row runs, so writing it to
// global memory directly means one 1- or 2-byte store per value, 64 bytes per
// half-wave at best; the SwiGLU backward also needs the saved g and u of
// every value.  Both cost more than the tile's MFMAs at these shapes.  Here
// the tile goes through LDS instead, in the two 64 KB operand buffers, free
// once the K loop is done.  bf16 results are staged as column runs (4 rows
// of one column per 8-byte chunk, written with one LDS store per 4 values)
// and read back as rows with gfx950's transposing LDS read; the fp32 staging
// of the MX epilogue and the SwiGLU backward's g, u span use row-major
// planes, each row a whole number of 16-byte chunks with the chunk index
// XOR-ed by the row (the accumulator layout's row pairs r, r + 4 then fall
// in different bank groups).  All 256 threads then copy rows out, 16 bytes
// per lane: full 128-byte lines.
#pragma once

#include "gemm_common.h"
#include "mx_device.h"

namespace moe {

// Byte offset of 16-byte chunk `ch` of row `r` in a plane whose rows hold
// `nch` chunks (a power of two).
__device__ __forceinline__ int st_off(int r, int ch, int nch) {
  return (r * nch + (ch ^ (r & (nch - 1)))) << 4;
}

// Byte offset of byte `b` of row `r`.
__device__ __forceinline__ int st_byte(int r, int b, int nch) {
  return st_off(r, b >> 4, nch) + (b & 15);
}

// Row (within its 128-row plane) of accumulator element v of 32-row block i.
__device__ __forceinline__ int acc_row(int i, int v, int lane) {
  return 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// Tile geometry handed to the epilogues.
struct TileAt {
  int m0, n0, rowbase, Mg, wm0, wn0, lane, tid;
};

// ---- Column-run staging of bf16 tiles
//
// Per 32 x 32 block, a lane's accumulators are runs of 4 consecutive rows of
// one column.  Staged as bf16, a run is one 8-byte chunk: chunk (q, c) holds
// rows 4q .. 4q+3 of column c at byte (q ncol + (c ^ ((c >> 2) & 4))) * 8 of a
// plane of ncol columns, so a lane stages 4 values with one 8-byte LDS write
// after two packed conversions.  The copy-out reads the runs back with
// ds_read_b64_tr_b16, gfx950's transposing LDS read: within each 16-lane
// group, output lane 4a + b receives element b of the 8-byte chunks
// addressed by lanes a, 4 + a, 8 + a and 12 + a (measured on MI355X).  When
// group lane 4s + a addresses column c + 8a + s of row quad q, output lane
// 4a + b therefore receives row 4q + b, columns c + 8a .. c + 8a + 3, and a
// second read four columns on gives the next four: a 16-byte row chunk per
// lane, and for each row 16 lanes x 16 bytes of consecutive columns.  The XOR
// of column bit 4 into bit 2 puts the 16 chunks of one group's read, and the
// 16 chunks of one half-wave's write, in distinct banks.

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 *lds_v4i16_t;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int run_off(int q, int c, int ncol) {
  return (q * ncol + (c ^ ((c >> 2) & 4))) << 3;
}

// Two fp32 values as packed bf16, round to nearest even (v_cvt_pk_bf16_f32;
// the same rounding as f32_to_bf16).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// The wave's 128 x 128 accumulators as bf16 runs into its plane (128 rows x
// 256 columns: the wave's rows are plane rows 0-127, its columns wn0 + ...).
__device__ __forceinline__ void stage_acc_runs(uint8_t *plane, const f32x16 (&acc)[4][4],
                                               int wn0, int lane) {
  const int qh = lane >> 5, c = wn0 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int vq = 0; vq < 4; vq++) {
        const uint2 w = make_uint2(cvt_pk_bf16(acc[i][j][4 * vq], acc[i][j][4 * vq + 1]),
                                   cvt_pk_bf16(acc[i][j][4 * vq + 2], acc[i][j][4 * vq + 3]));
        *(uint2 *)(plane + run_off(8 * i + 2 * vq + qh, c + 32 * j, 256)) = w;
      }
}

// Copies a run-staged plane (nq row quads x ncol columns, ncol a multiple of
// 128) to a row-major bf16 matrix dst (pitch ld elements): rows below
// rows_valid, columns below col_valid (a multiple of 8).  Units of (row quad,
// 128 columns) go to the four waves in turn; each wave reads eight units
// before it stores them.
__device__ __forceinline__ void copy_runs_out(const uint8_t *plane, int ncol, int nq,
                                              int rows_valid, int col_valid, uint16_t *dst,
                                              long ld, int wave, int lane) {
  constexpr int B = 8;
  const int g = lane >> 4, y = lane & 15;
  const int rc = 32 * g + 8 * (y & 3) + (y >> 2);  // column this lane addresses
  const int oc = 32 * g + 8 * (y >> 2), orow = y & 3;  // what it receives
  const int ncb = ncol >> 7, units = nq * ncb;
  for (int u0 = wave; u0 < units; u0 += 4 * B) {
    v4i16 lo[B], hi[B];
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int u = min(u0 + 4 * k, units - 1);
      const int q = u / ncb, cb = (u - q * ncb) << 7;
      lo[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t)(plane + run_off(q, cb + rc, ncol)));
      hi[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t)(plane + run_off(q, cb + rc + 4, ncol)));
    }
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int u = u0 + 4 * k;
      const int q = u / ncb, cb = (u - q * ncb) << 7;
      const int row = 4 * q + orow, col = cb + oc;
      if (u < units && row < rows_valid && col < col_valid) {
        const uint2 l = __builtin_bit_cast(uint2, lo[k]), h = __builtin_bit_cast(uint2, hi[k]);
        *(uint4 *)(dst + (size_t)row * ld + col) = make_uint4(l.x, l.y, h.x, h.y);
      }
    }
  }
}

// One eighth of the SwiGLU backward's output (copy_runs_out over 32 rows x
// 512 packed columns, 8 row quads) with exactly 8 store instructions per
// wave whatever the valid rows and columns: a lane outside them stores to an
// offset past the buffer descriptor, which the hardware drops.  With no
// branch around a store the compiler counts them exactly, so a later wait
// for older loads can leave these 8 stores in flight (vmcnt counts stores).
__device__ __forceinline__ void copy_eighth_out(const uint8_t *plane, int rows_valid,
                                                int col_valid, uint16_t *dst, long ld, int wave,
                                                int lane) {
  constexpr int ncol = 512, ncb = ncol >> 7;
  const int g = lane >> 4, y = lane & 15;
  const int rc = 32 * g + 8 * (y & 3) + (y >> 2);  // column this lane addresses
  const int oc = 32 * g + 8 * (y >> 2), orow = y & 3;  // what it receives
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void *)dst, (short)0, 0x7FFFFFFF, kBufferDword3);
  v4i16 lo[8], hi[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int u = wave + 4 * k, q = u / ncb, cb = (u - q * ncb) << 7;
    lo[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t)(plane + run_off(q, cb + rc, ncol)));
    hi[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t)(plane + run_off(q, cb + rc + 4, ncol)));
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int u = wave + 4 * k, q = u / ncb, cb = (u - q * ncb) << 7;
    const int row = 4 * q + orow, col = cb + oc;
    const uint32_t off = row < rows_valid && col < col_valid
                             ? (uint32_t)((row * ld + col) * 2)
                             : 0x80000000u;
    const uint2 l = __builtin_bit_cast(uint2, lo[k]), h = __builtin_bit_cast(uint2, hi[k]);
    const v4u32 v = {l.x, l.y, h.x, h.y};
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, (int)off, 0, 0);
  }
}

// Both planes of a run-staged 256 x 256 tile out to C (pitch ldc), columns
// from c0, `cols` valid columns.
__device__ __forceinline__ void store_run_planes(const uint8_t *L0, const uint8_t *L1,
                                                 const TileAt &t, uint16_t *C, long ldc, long c0,
                                                 int cols) {
#pragma unroll
  for (int pl = 0; pl < 2; pl++) {
    const int r0 = t.m0 + 128 * pl;
    const int rv = min(128, t.Mg - r0);
    if (rv > 0)
      copy_runs_out(pl ? L1 : L0, 256, 32, rv, cols, C + (size_t)(t.rowbase + r0) * ldc + c0,
                    ldc, t.tid >> 6, t.lane);
  }
}

// EPI_BF16: C[rows][N] = bf16(acc).
__device__ __forceinline__ void tile_epi_bf16(const GemmArgs &p, const f32x16 (&acc)[4][4],
                                              uint8_t *L0, uint8_t *L1, const TileAt &t) {
  __syncthreads();
  stage_acc_runs(t.wm0 ? L1 : L0, acc, t.wn0, t.lane);
  __syncthreads();
  store_run_planes(L0, L1, t, (uint16_t *)p.C, p.ldc, t.n0, min(BN, p.N - t.n0));
}

// EPI_SWIGLU: packed columns hold 64-column blocks [32 gate | 32 up].
// C2 (optional) <- g|u as bf16; C <- a = silu(g) u as bf16, or with MX
// (mx->q_out) a quantised along I in 32-blocks: codes to q_out, scales to
// s_out, the round trip as bf16 to C.  For MX the tile's a values are staged
// as fp32 (a plane row = 128 values = 512 bytes) and each thread then
// converts whole 32-value blocks, so no cross-lane reduction is needed.
template <bool MX>
__device__ __forceinline__ void tile_epi_swiglu(const GemmArgs &p, const MxOperands *mx,
                                                const f32x16 (&acc)[4][4], uint8_t *L0,
                                                uint8_t *L1, const TileAt &t) {
  const int I = p.N / 2;
  uint8_t *plane = t.wm0 ? L1 : L0;
  __syncthreads();
  if (p.C2) {
    stage_acc_runs(plane, acc, t.wn0, t.lane);
    __syncthreads();
    store_run_planes(L0, L1, t, (uint16_t *)p.C2, p.ldc2, t.n0, min(BN, p.N - t.n0));
    __syncthreads();
  }
  const int ncol = t.lane & 31;
  const int a0 = t.n0 / 2, a_valid = min(BN / 2, I - a0);
  if constexpr (!MX) {
    // a as bf16 runs: one plane (L0) of 256 rows x 128 columns
    const int qh = t.lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int jj = 0; jj < 2; jj++) {
        const int ca = t.wn0 / 2 + 32 * jj + ncol;  // tile-local a column
#pragma unroll
        for (int vq = 0; vq < 4; vq++) {
          float av[4];
#pragma unroll
          for (int e = 0; e < 4; e++)
            av[e] = silu_f(acc[i][2 * jj][4 * vq + e]) * acc[i][2 * jj + 1][4 * vq + e];
          const uint2 w = make_uint2(cvt_pk_bf16(av[0], av[1]), cvt_pk_bf16(av[2], av[3]));
          *(uint2 *)(L0 + run_off((t.wm0 >> 2) + 8 * i + 2 * vq + qh, ca, 128)) = w;
        }
      }
    __syncthreads();
    copy_runs_out(L0, 128, 64, min(BM, t.Mg - t.m0), a_valid,
                  (uint16_t *)p.C + (size_t)(t.rowbase + t.m0) * p.ldc + a0, p.ldc, t.tid >> 6,
                  t.lane);
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int jj = 0; jj < 2; jj++) {
        const int ca = t.wn0 / 2 + 32 * jj + ncol;  // tile-local a column
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int r = acc_row(i, v, t.lane);
          const float av = silu_f(acc[i][2 * jj][v]) * acc[i][2 * jj + 1][v];
          *(float *)(plane + st_byte(r, 4 * ca, 32)) = av;
        }
      }
    __syncthreads();
    // 256 rows x 4 blocks of 32 values; 4 consecutive threads take one row
#pragma unroll
    for (int it = 0; it < 4; it++) {
      const int q = t.tid + NT * it;
      const int row = q >> 2, blk = q & 3;
      const int grow_local = t.m0 + row;
      if (grow_local >= t.Mg || blk * 32 >= a_valid) continue;
      const uint8_t *pl = row < 128 ? L0 : L1;
      const int r = row & 127;
      float v[32];
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const float4 f = *(const float4 *)(pl + st_off(r, blk * 8 + c, 32));
        v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
      }
      uint32_t w[8];
      float deq[32];
      const uint32_t sc = mx_block32(v, w, deq);
      const size_t grow = (size_t)(t.rowbase + grow_local);
      uint4 *dq = (uint4 *)(mx->q_out + grow * I + a0 + blk * 32);
      dq[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dq[1] = make_uint4(w[4], w[5], w[6], w[7]);
      uint4 *dh = (uint4 *)((uint16_t *)p.C + grow * p.ldc + a0 + blk * 32);
#pragma unroll
      for (int c = 0; c < 4; c++) dh[c] = pack8(deq + 8 * c);
      const int b = a0 / 32 + blk;  // 32-block of a along I; scales K-blocked
      mx->s_out[((size_t)(b >> 2) * mx->a_rows + grow) * 4 + (b & 3)] = (uint8_t)sc;
    }
  }
}

// EPI_SWIGLU_BWD: the GEMM gives dA for intermediate columns; with the saved
// g|u (p.aux, packed like the forward's C2) it writes dg|du (packed the same
// way) to C:  dg = dA u silu'(g),  du = dA silu(g),
// silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).
// The tile's 256 intermediate columns own a 512-column (1 KB) g|u span per
// row.  The tile is done in eighths of 32 rows, software-pipelined over four
// 32 KB LDS regions (P0, P1 in L0; Q0, Q1 in L1).  For eighth e:
//  - its g|u rows arrive in Q[e & 1] by direct-to-LDS DMA, issued while
//    eighth e - 1 is computed (row r in bytes [1024 r, 1024 r + 1024),
//    16-byte chunk ch at slot ch ^ 2 (r & 3));
//  - the two waves that own its rows write their fp32 dA as 4-row runs into
//    P[e & 1] (16 bytes per run, run (q, c) at byte (256 q + c) * 16);
//  - all four waves take runs in turn: a transposing read of Q gives a lane
//    the 4-row runs of g and of u of its column (group lane 4s + a
//    addresses row 4q + s at packed column pg(C) + 4a, so output lane
//    4a + b holds column C + 4a + b), one 16-byte read its dA run; dg and
//    du go back into P[e & 1] as bf16 runs once every dA run is read;
//  - its rows are copied out with the transposing read while eighth e + 1
//    is computed.
// Every SIMD does a quarter of the sigmoid arithmetic.

// Byte offset in a Q region of the 8-byte piece at packed column pc (a
// multiple of 4) of row r.
__device__ __forceinline__ int gu_off(int r, int pc) {
  return (r << 10) + ((((pc >> 3) ^ ((r & 3) << 1))) << 4) + (((pc >> 2) & 1) << 3);
}

// Packed g column of intermediate column c: 64-column blocks [32 g | 32 u].
__device__ __forceinline__ int packed_g(int c) { return ((c >> 5) << 6) + (c & 31); }

constexpr int kBwdRegion = 32 * 1024;

__device__ __forceinline__ void tile_epi_swiglu_bwd(const GemmArgs &p,
                                                    const f32x16 (&acc)[4][4], uint8_t *L0,
                                                    uint8_t *L1, const TileAt &t) {
  const int span_cols = min(2 * BN, 2 * (p.N - t.n0));  // valid packed columns
  const int wave = t.tid >> 6, lane = t.lane;
  const int g = lane >> 4, y = lane & 15;
  const int rs4 = y >> 2, ra = y & 3;  // transposing read: row offset, column quad
  const uint16_t *gu_base = p.aux + (size_t)(t.rowbase + t.m0) * p.ldaux + 2L * t.n0;
  uint16_t *out_base = (uint16_t *)p.C + (size_t)(t.rowbase + t.m0) * p.ldc + 2L * t.n0;
  auto rows_of = [&](int e) { return min(32, t.Mg - t.m0 - 32 * e); };
  // Q[e & 1] holds eighth e's g|u rows: the even eighths in L1, the odd ones
  // in an LDS object of their own (32 KB more, 160 KB in all).  The compiler
  // waits for the DMAs into an LDS object before reading it, so with both
  // halves in L1 every read of eighth e also waited for eighth e + 1's DMA,
  // issued just before.
  __shared__ __attribute__((aligned(1024))) uint8_t q_odd[kBwdRegion];
  auto q_of = [&](int e) { return (e & 1) ? q_odd : L1; };
  // g|u rows of eighth e into Q[e & 1] (rows past the tile read as zeros)
  auto dma = [&](int e) {
    const int rv = rows_of(e);
    if (rv <= 0) return;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(gu_base + (size_t)32 * e * p.ldaux), (short)0, rv * (int)p.ldaux * 2,
        kBufferDword3);
    uint8_t *Q = q_of(e);
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int r = wave * 8 + k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_ptr_t)(Q + (r << 10)), 16,
          (uint32_t)(r * (int)p.ldaux * 2 + ((lane ^ ((r & 3) << 1)) << 4)), 0, 0, 0);
    }
  };
  // 8 store instructions per wave, also for rows past the tile (dropped)
  auto copy_out = [&](int e) {
    copy_eighth_out(L0 + (e & 1) * kBwdRegion, max(rows_of(e), 0), span_cols,
                    out_base + (size_t)32 * e * p.ldc, p.ldc, wave, lane);
  };
  // The barriers below are lds_barrier: __syncthreads' fence would also wait
  // for the next eighth's g|u DMA (issued just before) and the previous
  // eighth's stores, every eighth.  Only the wait at the top of an eighth
  // waits for memory: for this wave's DMA of the eighth's rows, which was
  // followed only by the 8 stores of copy_out(e - 2), which stay in flight.
  __syncthreads();  // the operand buffers are free
  dma(0);
#pragma unroll
  for (int e = 0; e < 8; e++) {
    uint8_t *P = L0 + (e & 1) * kBwdRegion;
    const uint8_t *Q = q_of(e);
    const int rv = rows_of(e);
    if (e >= 2)  // (e is a constant once the loop is unrolled)
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(8));  // eighth e's rows
    else
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    lds_barrier();
    if (e + 1 < 8) dma(e + 1);  // Q[(e + 1) & 1] was last read by eighth e - 1
    if (rv > 0 && t.wm0 == 128 * (e >> 2)) {
      const int i = e & 3, qh = lane >> 5;
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int vq = 0; vq < 4; vq++) {
          const int c = t.wn0 + 32 * j + (lane & 31);
          *(float4 *)(P + (((2 * vq + qh) * 256 + c) << 4)) =
              make_float4(acc[i][j][4 * vq], acc[i][j][4 * vq + 1], acc[i][j][4 * vq + 2],
                          acc[i][j][4 * vq + 3]);
        }
    }
    lds_barrier();
    // runs: wave w takes units w, w + 4 (8 each): row quad u / 4, 64 columns
    // (u % 4) * 64, group g their 16 columns from 16 g
    uint2 og[8], ou[8];
    if (rv > 0) {
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int u = wave + 4 * k, q = u >> 2;
        const int C = ((u & 3) << 6) + 16 * g, c = C + y;
        const int pr = packed_g(C) + 4 * ra;
        const v4i16 gr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t)(Q + gu_off(4 * q + rs4, pr)));
        const v4i16 ur = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t)(Q + gu_off(4 * q + rs4, pr + 32)));
        const float4 da = *(const float4 *)(P + ((q * 256 + c) << 4));
        const float dav[4] = {da.x, da.y, da.z, da.w};
        float dg[4], du[4];
#pragma unroll
        for (int x = 0; x < 4; x++) {
          const float gv = __uint_as_float((uint32_t)(uint16_t)gr[x] << 16);
          const float uv = __uint_as_float((uint32_t)(uint16_t)ur[x] << 16);
          const float sg = sigmoid_f(gv);
          dg[x] = dav[x] * uv * sg * (1.0f + gv * (1.0f - sg));
          du[x] = dav[x] * gv * sg;
        }
        og[k] = make_uint2(cvt_pk_bf16(dg[0], dg[1]), cvt_pk_bf16(dg[2], dg[3]));
        ou[k] = make_uint2(cvt_pk_bf16(du[0], du[1]), cvt_pk_bf16(du[2], du[3]));
      }
    }
    if (e > 0) copy_out(e - 1);
    lds_barrier();  // every dA run of eighth e has been read
    if (rv > 0) {
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int u = wave + 4 * k, q = u >> 2;
        const int c = ((u & 3) << 6) + 16 * g + y;
        *(uint2 *)(P + run_off(q, packed_g(c), 512)) = og[k];
        *(uint2 *)(P + run_off(q, packed_g(c) + 32, 512)) = ou[k];
      }
    }
  }
  lds_barrier();
  copy_out(7);
}

}  // namespace moe
