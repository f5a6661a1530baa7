// Host-side launchers of libmoe's kernels (all asynchronous on stream `s`).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kLayoutChunk = 1024;  // flat rows per block of the layout passes
constexpr int kTileM = 256;         // rows of one grouped-GEMM tile
constexpr int kTileN = 256;         // columns of one grouped-GEMM tile
constexpr int kTileK = 64;          // contraction depth of one LDS stage
constexpr int kPipeMaxMinibatches = 1024;  // minibatches of one pipelined call, at most
constexpr int kMaxTopKList = 16;    // top-k bound of the token-list kernels

// route_layout.hip
void launch_topk(const float *logits, int T, int E, int k, int32_t *idx, float *w,
                 hipStream_t s);
void launch_layout(const int32_t *idx, int R, int E, int32_t *chunk_counts, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *tile_start,
                   int tile_rows, int32_t *order, hipStream_t s);
void launch_dense_groups(int32_t *offsets, int32_t *tile_start, int32_t *order, int M,
                         int tile_rows, hipStream_t s);
void launch_tile_starts(const int32_t *offsets, int G, int tile_rows, int32_t *tile_start,
                        hipStream_t s);
void launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s);

// permute.hip
void launch_dispatch_bf16(const uint16_t *x, const int32_t *perm, uint16_t *xp, int R, int k,
                          int H, hipStream_t s);
void launch_dispatch_mx(const uint16_t *x, const int32_t *perm, uint8_t *xq, uint8_t *xs,
                        uint16_t *xhat, int R, int k, int H, hipStream_t s);
// Scatter forms (token-driven, need inv = perm^-1): same outputs as above.
void launch_dispatch_push_bf16(const uint16_t *x, const int32_t *inv, uint16_t *xp, int T, int k,
                               int H, hipStream_t s);
void launch_dispatch_push_mx(const uint16_t *x, const int32_t *inv, uint8_t *xq, uint8_t *xs,
                             uint16_t *xhat, int T, int k, int H, hipStream_t s);
// ... writing only the sorted rows in [r0, r1) (one minibatch)
void launch_dispatch_push_bf16_range(const uint16_t *x, const int32_t *inv, uint16_t *xp, int T,
                                     int k, int H, int r0, int r1, hipStream_t s);
void launch_dispatch_push_mx_range(const uint16_t *x, const int32_t *inv, uint8_t *xq,
                                   uint8_t *xs, uint16_t *xhat, int T, int k, int H, int r0,
                                   int r1, hipStream_t s);
void launch_quant_rows_mx(const uint16_t *src, int rows, int cols, uint8_t *q, uint8_t *sc,
                          hipStream_t s);
// Rows [row0, row0 + rows) of a matrix of rows_total rows (scale plane stride).
void launch_dispatch_mx_range(const uint16_t *x, const int32_t *perm, uint8_t *xq, uint8_t *xs,
                              uint16_t *xhat, int row0, int rows, int rows_total, int k, int H,
                              hipStream_t s);
void launch_quant_rows_mx_range(const uint16_t *src, int row0, int rows, int rows_total, int cols,
                                uint8_t *q, uint8_t *sc, hipStream_t s);
void launch_combine(const uint16_t *y, const float *w, const int32_t *inv, const uint16_t *ys,
                    uint16_t *out, int T, int k, int H, hipStream_t s);
// dyq/dys non-null (MXFP8): dY is also written as E4M3 codes [T k][H] and
// K-blocked E8M0 scales, exactly as launch_quant_rows_mx would make them.
void launch_reverse_combine(const uint16_t *dout, const uint16_t *y, const float *w,
                            const int32_t *inv, uint16_t *dy, float *dw, float *dsel, int T,
                            int k, int H, uint8_t *dyq, uint8_t *dys, hipStream_t s);
void launch_reverse_dispatch(const uint16_t *dX, const int32_t *inv, const int32_t *idx,
                             const float *dsel, const uint16_t *wrT, const uint16_t *dxs,
                             uint16_t *dx, int T, int k, int H, hipStream_t s);
void launch_router_wgrad(const uint16_t *x, const int32_t *perm, const int32_t *offsets,
                         const float *dsel, float *dwr, int E, int k, int H, hipStream_t s);
void launch_transpose_pack(const uint16_t *in, uint16_t *out, int G, int rows, int cols,
                           int out_rows_total, int blk_stride, int blk_off, hipStream_t s);
void launch_interleave_copy(const uint16_t *in, uint16_t *out, int G, int rows, int cols,
                            int out_cols, int blk_stride, int blk_off, hipStream_t s);

// pipeline.hip: the minibatch schedule's plan and its per-minibatch data movement
void launch_pipe_offsets(const int32_t *offsets, int E, int R, int MB, int NM, int32_t *moff,
                         int32_t *mts, hipStream_t s);
void launch_pipe_lists(const int32_t *inv, int T, int k, int R, int MB, int NM, bool last,
                       int32_t *tl, int32_t *tl_off, hipStream_t s);
void launch_combine_list(const uint16_t *y, const float *w, const int32_t *inv,
                         const uint16_t *ys, uint16_t *out, const int32_t *tl,
                         const int32_t *tl_off, int m, int T, int k, int H, hipStream_t s);
void launch_reverse_combine_rows(const uint16_t *dout, const uint16_t *y, const float *w,
                                 const int32_t *perm, uint16_t *dy, float *dw, int r0, int rows,
                                 int k, int H, uint8_t *dyq, uint8_t *dys, long rows_total,
                                 hipStream_t s);
void launch_reverse_dispatch_list(const uint16_t *dX, const int32_t *inv, const int32_t *idx,
                                  const float *w, const float *dw, float *dsel,
                                  const uint16_t *wrT, const uint16_t *dxs, uint16_t *dx,
                                  const int32_t *tl, const int32_t *tl_off, int m, int T, int k,
                                  int H, hipStream_t s);

// decode.hip: few-token expert FFN (weight-streaming GEMV form).  For each of
// G groups (experts; offsets [G+1]) and its rows r: act[r] = silu(x[t] Wg) *
// (x[t] Wu), y[r] = act[r] Wd, t = perm[r] / k (perm == nullptr: t = r).
// guT: packed gate/up [G][2I][H]; dT: packed down [G][H][I].  `rows`: the
// rows over all groups (bounds the rows of one group).
void launch_decode_ffn(const uint16_t *x, const int32_t *perm, const int32_t *offsets, int G,
                       long rows, int k, int H, int I, const uint16_t *guT, const uint16_t *dT,
                       uint16_t *act, uint16_t *y, hipStream_t s);
// The layer's layout (counts, offsets, perm, inv; same result as
// launch_layout) in one workgroup, for R <= kDecLayoutMax routed rows.
constexpr int kDecLayoutMax = 1024;
void launch_decode_layout(const int32_t *idx, int R, int E, int32_t *counts, int32_t *offsets,
                          int32_t *perm, int32_t *inv, hipStream_t s);

// gemm.hip: grouped GEMMs on MFMA (bf16 inputs, fp32 accumulation)
enum EpiKind { EPI_BF16 = 0, EPI_F32 = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3, EPI_WGRAD_GU = 4 };

struct GemmArgs {
  const uint16_t *A;
  long lda;
  const uint16_t *B;
  long ldb;
  long sB;          // per-group stride of B (row-ragged mode)
  void *C;
  long ldc;
  long sC;          // per-group stride of C (weight-gradient mode)
  void *C2;         // second output (SwiGLU: saved g|u; dW_up in weight-gradient mode)
  long ldc2;
  const uint16_t *aux;  // SwiGLU backward: saved g|u
  long ldaux;
  const float *bias;    // EPI_F32: optional per-column bias
  const int32_t *offsets;     // [G+1] group row offsets
  const int32_t *tile_start;  // [G+1] prefix of row tiles (row-ragged mode)
  const int32_t *order;       // [G] group processing order (weight-gradient mode)
  int G, M, N, K;
  int n_tiles_m, n_tiles_n;
  int xcd_major;  // weight-gradient mode: XCD-major tile order (gemm_tn_kernel)
  unsigned long long *stamps;  // optional per-tile timing counters (TileClock)
};

// Counter block of the in-kernel timing of a stage's GEMM tiles (device,
// 8 words, zeroed by the caller): every tile adds, from thread 0 of its
// workgroup, the words below.  Shader cycles from s_memtime, real time from
// the 100 MHz s_memrealtime, so cycles / ticks * 100 MHz is the clock the
// tiles ran at.
enum {
  kStampTiles = 0,      // tiles
  kStampCycles = 1,     // shader cycles, tile start to epilogue end
  kStampLoop = 2,       // of which prologue + K loop
  kStampEpilogue = 3,   // of which epilogue
  kStampTicks = 4,      // real-time ticks (100 MHz), tile start to end
  kStampWords = 8
};

// The counter block the GEMMs launched now add to (nullptr = none): set by
// the layer call for the stage it is enqueueing (host, per thread).
unsigned long long *current_stamps();

// Row-ragged grouped GEMM: for group g, rows [offsets[g], offsets[g+1]) of A
// (K-contiguous, [rows][K]) times B_g (K-contiguous [N][K], or N-contiguous
// [K][N] when b_kcontig is false) -> epilogue.  `max_rows` bounds the total
// number of rows (sizes the grid).
void launch_gemm_rows(const GemmArgs &p, int epi, bool b_kcontig, int max_rows, hipStream_t s);

// Row-ragged grouped GEMM on MXFP8 operands (E4M3 codes + E8M0 scales per 32
// along K): A codes [rows][K] with scales [rows][K/32]; B codes [G][N][K]
// with scales [G][N][K/32].  Epilogues: EPI_BF16, EPI_SWIGLU (with
// p.mx_out: a quantised along I into codes/scales, and its bf16 round trip
// into p.C), EPI_SWIGLU_BWD.
//
// E8M0 scales are stored K-blocked: for a matrix of `rows` rows, the scale of
// row r and 32-wide block b is byte (b/4 * rows + r) * 4 + b%4, i.e.
// [K/128][rows][4].  A GEMM stage (128 values of K) then finds the scales of
// a tile's consecutive rows in consecutive dwords.
// Element formats of an MX GEMM's B operand (the expert weights), as the
// f8f6f4 matrix instruction numbers them: E4M3 (MXFP8), FP6 E2M3, FP6 E3M2,
// FP4 E2M1.  A operands (activations, gradients) are always E4M3.
constexpr int kMxE4M3 = 0, kMxE2M3 = 2, kMxE3M2 = 3, kMxE2M1 = 4;

struct MxOperands {
  const uint8_t *a_scale;   // A scales, [K/128][a_rows][4]
  const uint8_t *b_scale;   // B scales, [K/128][G*N][4] (row g*N + n)
  int a_rows;               // rows of the A scale matrix
  uint8_t *q_out;           // SwiGLU MX epilogue: a codes [rows][I]
  uint8_t *s_out;           // SwiGLU MX epilogue: a scales, [I/128][a_rows][4]
  int b_fmt = kMxE4M3;      // B element format (kMx*); E2M1 rows are K/2 bytes
};

// MX codes of a bf16 matrix [rows][K] quantised along K in a lower-precision
// element format (kMxE2M3, kMxE3M2, kMxE2M1), with the E8M0 scales K-blocked
// as for E4M3.  E2M1: 16 bytes per 32-value block, rows of K/2 bytes; FP6:
// 24 bytes of codes and 8 zero bytes per block, rows of K bytes.
void launch_quant_rows_mx_low(const uint16_t *src, int rows, int K, uint8_t *q, uint8_t *sc,
                              int fmt, hipStream_t s);
void launch_gemm_rows_mx(const GemmArgs &p, const MxOperands &mx, int epi, int max_rows,
                         hipStream_t s);

// MX weight gradients (gemm_mx.hip).  poff[e] = prefix of the expert row
// counts rounded up to 128 (launch_pad_offsets); launch_quant_cols_mx
// quantises src [R][C] bf16 down its rows in 32-row blocks per expert
// segment into transposed codes q [C][Rp] with K-blocked scales
// [Rp/128][C][4] (Rp: the row stride, a multiple of 128 >= poff[E]);
// launch_gemm_mx_wgrad: C_g[M][N] = A_g^T B_g with A = transposed codes
// [M][Rp], B = [N][Rp] (p.lda = p.ldb = Rp), group g's contraction range
// [poff[g], poff[g+1]) (p.offsets = poff), p.order, fp32 epilogue (EPI_F32
// or EPI_WGRAD_GU), mx.a_scale / mx.b_scale the two scale planes.
void launch_pad_offsets(const int32_t *offsets, int E, int32_t *poff, hipStream_t s);
void launch_quant_cols_mx(const uint16_t *src, int R, int C, const int32_t *offsets,
                          const int32_t *poff, int E, long Rp, uint8_t *q, uint8_t *sc,
                          hipStream_t s);
void launch_gemm_mx_wgrad(const GemmArgs &p, const MxOperands &mx, int epi, hipStream_t s);

// Weight-gradient grouped GEMM: for group g, C_g[M][N] = sum over rows
// [offsets[g], offsets[g+1]) of A[row][M]^T B[row][N] (both row-major with the
// summed rows outermost).
// Weight gradients C_g = A_g^T B_g over the groups' row ranges; `rows`: the
// rows over all groups (at most), which picks the tile order.
void launch_gemm_wgrad(const GemmArgs &p, int epi, long rows, hipStream_t s);

}  // namespace moe
