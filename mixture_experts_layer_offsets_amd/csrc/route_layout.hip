// Schedule step of the layer: top-k routing and the expert-contiguous layout.
//
// Sources: kucoin.com news flash "O MoK do Cursor alcança aumento de
// desempenho de 2,37x no NVIDIA GB300 NVL72", §01 (each token picks a few
// experts; the system counts the tokens of every expert, decides where they
// go and keeps one expert's rows together for the grouped GEMM) and §02 (no
// CPU in the loop: everything is decided by GPU state).
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k + renormalised softmax.  One wave per token; each lane holds up to
// EPL logits (expert e sits in lane e % 64, slot e / 64).  k rounds of a
// wave arg-max under the total order (larger logit first, then lower index)
// select the experts; slot j's result is parked in lane j.

template <int EPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float *__restrict__ logits, int T, int E, int k,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[EPL];
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i++) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[(size_t)t * E + e] : 0.0f;
    taken[i] = e >= E;
  }
  float sel_v = 0.0f;
  int sel_e = 0;
  for (int j = 0; j < k; j++) {
    float bv = 0.0f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      const int e = lane + 64 * i;
      if (!taken[i] && (be == 0x7FFFFFFF || v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) {
#pragma unroll
      for (int i = 0; i < EPL; i++)
        if (i == (be >> 6)) taken[i] = true;
    }
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
  }
  const float m = __shfl(sel_v, 0, 64);
  const float ex = lane < k ? expf(sel_v - m) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = sel_e;
    w_out[(size_t)t * k + lane] = ex / s;
  }
}

void launch_topk(const float *logits, int T, int E, int k, int32_t *idx, float *w,
                 hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(topk_softmax_kernel<1>, grid, block, 0, s, logits, T, E, k, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_softmax_kernel<4>, grid, block, 0, s, logits, T, E, k, idx, w);
  else
    hipLaunchKernelGGL(topk_softmax_kernel<16>, grid, block, 0, s, logits, T, E, k, idx, w);
}

// ---------------------------------------------------------------------------
// Layout: a three-pass stable counting sort over the R = T*k flat rows.
//   count  : per-chunk histogram (kLayoutChunk rows per block)
//   scan   : per-expert totals, exclusive prefix over experts (offsets), the
//            per-(chunk, expert) starting rows, grouped-GEMM tile prefixes
//            and the experts ordered by load
//   scatter: stable rank of every row inside its chunk (wave ballots, then
//            wave and round prefixes in LDS) -> perm / inv_perm
// Every step is integer-only and order-fixed: the result does not depend on
// scheduling.  Expert ids are clamped into [0, E) so that a bad id can never
// address memory outside the outputs.

__device__ __forceinline__ int clamp_e(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void layout_count_kernel(const int32_t *__restrict__ idx,
                                                           int R, int E,
                                                           int32_t *__restrict__ chunk_counts) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kLayoutChunk;
  for (int i = threadIdx.x; i < kLayoutChunk; i += 256) {
    const int f = base + i;
    if (f < R) atomicAdd(&cnt[clamp_e(idx[f], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One block of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void layout_scan_kernel(
    int32_t *__restrict__ chunk_counts /* in: counts, out: starting rows */, int nchunks, int E,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ tile_start,
    int tile_rows, int32_t *__restrict__ order) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t st[1024];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; c++) {
      const size_t at = (size_t)c * E + e;
      const int n = chunk_counts[at];
      chunk_counts[at] = total;
      total += n;
    }
  }
  const int tiles = (total + tile_rows - 1) / tile_rows;
  sc[e] = e < E ? total : 0;
  st[e] = e < E ? tiles : 0;
  __syncthreads();
  // inclusive Hillis-Steele scans over experts
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = e >= o ? sc[e - o] : 0;
    const int b = e >= o ? st[e - o] : 0;
    __syncthreads();
    sc[e] += a;
    st[e] += b;
    __syncthreads();
  }
  if (e < E) {
    const int start = sc[e] - total;
    counts[e] = total;
    offsets[e] = start;
    tile_start[e] = st[e] - tiles;
    if (e == E - 1) {
      offsets[E] = sc[e];
      tile_start[E] = st[e];
    }
    for (int c = 0; c < nchunks; c++) chunk_counts[(size_t)c * E + e] += start;
    // rank by (load descending, index ascending)
    int rank = 0;
    for (int o = 0; o < E; o++) {
      const int n = sc[o] - (o ? sc[o - 1] : 0);
      rank += (n > total) || (n == total && o < e);
    }
    order[rank] = e;
  }
}

__global__ __launch_bounds__(256) void layout_scatter_kernel(
    const int32_t *__restrict__ idx, int R, int E, const int32_t *__restrict__ chunk_start,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
  extern __shared__ int32_t sm[];
  int32_t *run = sm;          // [E] next free row of each expert for this chunk
  int32_t *wcnt = sm + E;     // [4][E] rows of each expert per wave in this round
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) {
    run[e] = chunk_start[(size_t)blockIdx.x * E + e];
    wcnt[e] = wcnt[E + e] = wcnt[2 * E + e] = wcnt[3 * E + e] = 0;
  }
  __syncthreads();
  const int base = blockIdx.x * kLayoutChunk;
  for (int round = 0; round < kLayoutChunk / 256; round++) {
    const int f = base + round * 256 + tid;
    const bool valid = f < R;
    const int e = valid ? clamp_e(idx[f], E) : -1;
    // lanes of this wave that share my expert
    uint64_t active = __ballot(valid);
    uint64_t mine = 0;
    while (active) {
      const int leader = __ffsll((unsigned long long)active) - 1;
      const int el = __shfl(e, leader, 64);
      const uint64_t m = __ballot(valid && e == el) & active;
      if (valid && e == el) mine = m;
      active &= ~m;
    }
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int rank = __popcll(mine & below);
    const bool lead = valid && rank == 0;
    const int n = __popcll(mine);
    if (lead) wcnt[wave * E + e] = n;
    __syncthreads();
    if (valid) {
      int pos = run[e] + rank;
      for (int w = 0; w < wave; w++) pos += wcnt[w * E + e];
      perm[pos] = f;
      inv[f] = pos;
    }
    __syncthreads();
    if (lead) {
      atomicAdd(&run[e], n);
      wcnt[wave * E + e] = 0;
    }
    __syncthreads();
  }
}

void launch_layout(const int32_t *idx, int R, int E, int32_t *chunk_counts, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *tile_start,
                   int tile_rows, int32_t *order, hipStream_t s) {
  const int nchunks = (R + kLayoutChunk - 1) / kLayoutChunk;
  if (nchunks > 0)
    hipLaunchKernelGGL(layout_count_kernel, dim3(nchunks), dim3(256), E * sizeof(int32_t), s,
                       idx, R, E, chunk_counts);
  hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, E,
                     counts, offsets, tile_start, tile_rows, order);
  if (nchunks > 0)
    hipLaunchKernelGGL(layout_scatter_kernel, dim3(nchunks), dim3(256),
                       5 * E * sizeof(int32_t), s, idx, R, E, chunk_counts, perm, inv);
}

// Tile prefix of row-ragged groups given only their offsets (one block,
// thread g owns group g; G <= 1024): tile_start[g] = sum_{g'<g} ceil(n_g'/tile_rows).
__global__ __launch_bounds__(1024) void tile_starts_kernel(const int32_t *__restrict__ offsets,
                                                           int G, int tile_rows,
                                                           int32_t *__restrict__ tile_start) {
  __shared__ int32_t st[1024];
  const int g = threadIdx.x;
  const int tiles = g < G ? (offsets[g + 1] - offsets[g] + tile_rows - 1) / tile_rows : 0;
  st[g] = tiles;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int b = g >= o ? st[g - o] : 0;
    __syncthreads();
    st[g] += b;
    __syncthreads();
  }
  if (g < G) {
    tile_start[g] = st[g] - tiles;
    if (g == G - 1) tile_start[G] = st[g];
  }
}

void launch_tile_starts(const int32_t *offsets, int G, int tile_rows, int32_t *tile_start,
                        hipStream_t s) {
  hipLaunchKernelGGL(tile_starts_kernel, dim3(1), dim3(1024), 0, s, offsets, G, tile_rows,
                     tile_start);
}

__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
}

// Groups for a dense operand (the shared expert): one group of M rows.
__global__ void dense_groups_kernel(int32_t *offsets, int32_t *tile_start, int32_t *order, int M,
                                    int tile_rows) {
  if (threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = M;
    tile_start[0] = 0;
    tile_start[1] = (M + tile_rows - 1) / tile_rows;
    order[0] = 0;
  }
}

void launch_dense_groups(int32_t *offsets, int32_t *tile_start, int32_t *order, int M,
                         int tile_rows, hipStream_t s) {
  hipLaunchKernelGGL(dense_groups_kernel, dim3(1), dim3(64), 0, s, offsets, tile_start, order, M,
                     tile_rows);
}

}  // namespace moe
