// The layer forward as one persistent, pipelined kernel.
//
// The pages overlap the layer's communication with its expert GEMMs inside
// one kernel: a few processors move rows while the rest run GEMM tiles, the
// routed rows are cut into minibatches that flow through a bounded on-device
// buffer, completion is signalled by per-slot flags rather than host
// synchronisation, and the combine of one batch overlaps the dispatch of the
// next (kucoin.com news flash "O MoK do Cursor alcança aumento de desempenho
// de 2,37x no NVIDIA GB300 NVL72", §01-§03; deepdigest.ru article on MoK).
//
// On one MI355X the "communication" is the HBM gather of dispatch and the
// weighted gather of combine.  The grid is one workgroup per CU (each holds
// the 128 KB of LDS a GEMM tile needs, so all are co-resident on an idle
// GPU).  Workgroups [0, n_comm) serve the communication queue, the others the
// GEMM queue; both queues hand out tasks through an atomic counter in a fixed
// order, and every task waits only for tasks earlier in that order, so the
// schedule cannot deadlock.  Sorted routed rows are cut into minibatches of
// MB rows; per minibatch m:
//   D(m)  dispatch (gather, MXFP8 quantisation) of its rows, in chunks;
//   G1(m) gate/up GEMM + SwiGLU tiles of its rows (wait for D(m));
//   G2(m) down GEMM tiles (wait for all G1 tiles of the same row tile);
//   C(m)  combine of the tokens whose last routed row lies in minibatch m
//         (wait for G2 of every minibatch up to m, and the shared expert).
// Communication order: D(0..S-1), then D(m+S), C(m) for m = 0, 1, ...; D(m)
// for m >= S waits until G1(m-S) is complete, so at most S minibatches are
// in flight between dispatch and the GEMMs (the pages' S-slot ring; the rows
// themselves stay in the forward context, which the backward reads).
// GEMM order: the shared expert's tiles, then G1(0), G1(1), G2(0), G1(2),
// G2(1), ... The tiles and the combine are the same code as the staged
// kernels, so the outputs are bit-identical to the staged forward.
//
// Every wait is bounded (watchdog): a wait that exceeds its real-time budget sets
// the status word to MOE_ERR_DEVICE_TIMEOUT and the workgroup exits; the
// others then time out too, so the kernel always finishes.
#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"
#include "megakernel.h"
#include "row_tile.h"
#include "rows.h"

namespace moe {

namespace {

enum { PH_SG1 = 0, PH_SG2 = 1, PH_G1 = 2, PH_G2 = 3 };
enum { CP_D = 0, CP_C = 1 };

// Device-coherent load for polling.  Relaxed on purpose: an acquire load
// invalidates the XCD's whole L2 each time, and dozens of waves polling that
// way keep every L2 invalidating, which starves the producers being waited
// for.  The acquire fence is taken once, after the flag is seen.
__device__ __forceinline__ int ld_poll(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 100 MHz real-time counter (the watchdog's clock).
__device__ __forceinline__ unsigned long long now_ticks() {
  return __builtin_amdgcn_s_memrealtime();
}

// Stores of this workgroup become visible device-wide, then thread 0 adds
// `v` to the counter.
__device__ __forceinline__ void signal_add(int32_t *ctr, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(ctr, v);
}

struct Task {
  int kind, m, local, ok;
};

// Thread 0 takes the next task of a queue (phase table: kind, m, prefix);
// broadcast through LDS.
__device__ Task next_task(int32_t *ctr, const int32_t *ph_kind, const int32_t *ph_m,
                          const int32_t *ph_off, int nph, Task *sh) {
  if (threadIdx.x == 0) {
    Task t{0, 0, 0, 0};
    const int total = ph_off[nph];
    const int i = atomicAdd(ctr, 1);
    if (i < total) {
      int p = 0;
      while (ph_off[p + 1] <= i) p++;
      t = Task{ph_kind[p], ph_m[p], i - ph_off[p], 1};
    }
    *sh = t;
  }
  __syncthreads();
  const Task t = *sh;
  __syncthreads();
  return t;
}

// Thread 0 alone polls *flag until it reaches `target`, with sleeps that
// grow to ~2 us; the other waves wait at the barrier.  Every poll is a
// device-coherent load that leaves the XCD, and all of them hit the one line
// of counters that the producers' signalling atomics also need: with all 256
// threads of ~200 waiting workgroups polling every few hundred cycles, that
// line would see billions of requests per second, and the producers'
// signals and rows would queue behind them.  The status word is read every
// eighth poll.  A wait that outlasts the watchdog, or any wait after another
// workgroup reported a timeout, fails and leaves MOE_ERR_DEVICE_TIMEOUT in
// the status word; the workgroup then agrees on the outcome.
__device__ bool wait_all(const MkArgs &a, const int32_t *flag, int target, int *sh_fail) {
  if (threadIdx.x == 0) {
    const unsigned long long t0 = now_ticks();
    int fail = 0, nap = 1;
    for (int n = 0;; n++) {
      if (ld_poll(flag) >= target) break;
      if ((n & 7) == 7 &&
          (ld_poll(a.status) != MOE_OK || now_ticks() - t0 > a.watchdog_ticks)) {
        fail = 1;
        break;
      }
      for (int z = 0; z < nap; z++) __builtin_amdgcn_s_sleep(16);  // ~1000 cycles each
      nap = min(2 * nap, 4);
    }
    if (fail) atomicCAS(a.status, MOE_OK, MOE_ERR_DEVICE_TIMEOUT);
    *sh_fail = fail;
  }
  __syncthreads();
  const bool all_ok = *sh_fail == 0;
  __syncthreads();
  if (all_ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return all_ok;
}

template <bool MX>
__device__ void run_tile(const GemmArgs &p, const MxOperands &mx, int epi, int g, int m0, int n0,
                         int rowbase, int Mg, uint8_t *L0, uint8_t *L1) {
  if constexpr (MX) {
    if (epi == EPI_SWIGLU)
      mx_tile<EPI_SWIGLU>(p, mx, g, m0, n0, rowbase, Mg, L0, L1);
    else
      mx_tile<EPI_BF16>(p, mx, g, m0, n0, rowbase, Mg, L0, L1);
  } else {
    if (epi == EPI_SWIGLU)
      nt_tile<EPI_SWIGLU>(p, g, m0, n0, rowbase, Mg, (uint16_t *)L0, (uint16_t *)L1);
    else
      nt_tile<EPI_BF16>(p, g, m0, n0, rowbase, Mg, (uint16_t *)L0, (uint16_t *)L1);
  }
  __syncthreads();  // the LDS buffers are reused by the next tile
}

// Dispatch of sorted rows [r0, r1).
template <bool MX>
__device__ void dispatch_rows(const MkArgs &a, int r0, int r1) {
  const int HC = a.H / 8;
  const long n = (long)(r1 - r0) * HC;
  for (long id = threadIdx.x; id < n; id += NT) {
    const int r = r0 + (int)(id / HC), c = (int)(id % HC);
    const int src = a.perm[r] / a.k;
    const uint4 v = ((const uint4 *)a.x)[(size_t)src * HC + c];
    if constexpr (!MX) {
      ((uint4 *)a.x_perm)[(size_t)r * HC + c] = v;
    } else {
      // whole quads: n and the stride are multiples of 4
      float f[8], deq[8];
      unpack8(v, f);
      uint2 codes;
      const uint32_t sc = mx_quad8(f, &codes, deq);
      ((uint2 *)a.xq)[(size_t)r * HC + c] = codes;
      // scales K-blocked, as every consumer reads them: block b = c/4 of
      // row r at byte (b/4 * R + r) * 4 + b%4
      if ((c & 3) == 0) a.xs[((size_t)(c >> 4) * a.R + r) * 4 + ((c >> 2) & 3)] = (uint8_t)sc;
      ((uint4 *)a.x_perm)[(size_t)r * HC + c] = pack8(deq);
    }
  }
}

template <bool MX>
__global__ __launch_bounds__(NT, 1) void layer_fwd_megakernel(MkArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t L0[2 * BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t L1[2 * BM * 128];
  __shared__ Task sh_task;
  __shared__ int sh_fail;
  const int tid = threadIdx.x;
  const int nN1 = (2 * a.I + BN - 1) / BN, nN2 = (a.H + BN - 1) / BN;
  const int nN1s = (2 * a.Is + BN - 1) / BN;

  if ((int)blockIdx.x < a.n_comm) {
    // ---- communication workgroups
    for (;;) {
      const Task t = next_task(a.comm_next, a.cph_kind, a.cph_m, a.cph_off, a.n_cph, &sh_task);
      if (!t.ok) break;
      const int m = t.m;
      if (t.kind == CP_D) {
        if (m >= a.S) {
          const int need = (a.mt_off[m - a.S + 1] - a.mt_off[m - a.S]) * nN1;
          if (!wait_all(a, a.g1m_done + (m - a.S), need, &sh_fail)) return;
        }
        const int r0 = m * a.MB + t.local * a.DCH;
        const int r1 = min(min(r0 + a.DCH, (m + 1) * a.MB), a.R);
        dispatch_rows<MX>(a, r0, r1);
        signal_add(a.disp_done + m, 1);
      } else {
        // combine: every minibatch up to m and the shared expert complete
        for (int mm = 0; mm <= m; mm++) {
          const int need = (a.mt_off[mm + 1] - a.mt_off[mm]) * nN2;
          if (!wait_all(a, a.g2m_done + mm, need, &sh_fail)) return;
        }
        if (a.Is > 0 && !wait_all(a, a.sg2_done, ((a.T + BM - 1) / BM) * nN2, &sh_fail)) return;
        const int b0 = a.tl_off[m] + t.local * a.CT;
        const int b1 = min(b0 + a.CT, a.tl_off[m + 1]);
        const int HC = a.H / 8;
        for (int id = tid; id < (b1 - b0) * HC; id += NT) {
          const int tok = a.tl[b0 + id / HC], c = id % HC;
          combine8(a.y, a.w, a.inv, a.Is > 0 ? a.ys : nullptr, a.out, tok, c, a.k, HC);
        }
        __syncthreads();
      }
    }
    // the communication queue is done: help with GEMM tiles
  }

  // ---- GEMM workgroups
  for (;;) {
    const Task t = next_task(a.gemm_next, a.ph_kind, a.ph_m, a.ph_off, a.n_ph, &sh_task);
    if (!t.ok) break;
    if (t.kind == PH_SG1 || t.kind == PH_SG2) {
      const int nN = t.kind == PH_SG1 ? nN1s : nN2;
      const int mt = t.local / nN, nt = t.local % nN;
      if (t.kind == PH_SG2 && !wait_all(a, a.sg1_done + mt, nN1s, &sh_fail)) return;
      if (t.kind == PH_SG1)
        run_tile<MX>(a.sg1, a.smx1, EPI_SWIGLU, 0, mt * BM, nt * BN, 0, a.T, L0, L1);
      else
        run_tile<MX>(a.sg2, a.smx2, EPI_BF16, 0, mt * BM, nt * BN, 0, a.T, L0, L1);
      signal_add(t.kind == PH_SG1 ? a.sg1_done + mt : a.sg2_done, 1);
    } else {
      const int nN = t.kind == PH_G1 ? nN1 : nN2;
      const int idx = a.mt_off[t.m] + t.local / nN, nt = t.local % nN;
      const int e = a.mt_list[3 * idx], row0 = a.mt_list[3 * idx + 1],
                rows = a.mt_list[3 * idx + 2];
      if (t.kind == PH_G1) {
        const int chunks = (min((t.m + 1) * a.MB, a.R) - t.m * a.MB + a.DCH - 1) / a.DCH;
        if (!wait_all(a, a.disp_done + t.m, chunks, &sh_fail)) return;
        run_tile<MX>(a.g1, a.mx1, EPI_SWIGLU, e, 0, nt * BN, row0, rows, L0, L1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) {
          atomicAdd(a.g1_done + idx, 1);
          atomicAdd(a.g1m_done + t.m, 1);
        }
      } else {
        if (!wait_all(a, a.g1_done + idx, nN1, &sh_fail)) return;
        run_tile<MX>(a.g2, a.mx2, EPI_BF16, e, 0, nt * BN, row0, rows, L0, L1);
        signal_add(a.g2m_done + t.m, 1);
      }
    }
  }
}

// Plan of one call (one workgroup): the per-minibatch row tiles, the tokens
// ordered by the minibatch of their last routed row, both queues' phase
// tables, and zeroed counters.
__global__ __launch_bounds__(256) void mk_plan_kernel(MkArgs a) {
  __shared__ int cnt[kMkMaxMinibatches], fill[kMkMaxMinibatches];
  const int tid = threadIdx.x;
  for (int i = tid; i < a.n_counters; i += 256) a.counters[i] = 0;
  for (int m = tid; m < a.NM; m += 256) { cnt[m] = 0; fill[m] = 0; }
  __syncthreads();
  // tokens by last minibatch
  for (int t = tid; t < a.T; t += 256) {
    int last = 0;
    for (int j = 0; j < a.k; j++) last = max(last, a.inv[t * a.k + j]);
    const int m = last / a.MB;
    a.tok_m[t] = m;
    atomicAdd(&cnt[m], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int m = 0; m < a.NM; m++) { a.tl_off[m] = s; s += cnt[m]; }
    a.tl_off[a.NM] = s;
    // row tiles: minibatch rows cut at expert boundaries, 256 rows per tile
    int n = 0, e = 0;
    for (int m = 0; m < a.NM; m++) {
      a.mt_off[m] = n;
      int lo = m * a.MB;
      const int hi = min(a.R, lo + a.MB);
      while (lo < hi) {
        while (a.offsets[e + 1] <= lo) e++;
        const int end = min(hi, a.offsets[e + 1]);
        for (int r = lo; r < end; r += BM) {
          a.mt_list[3 * n] = e;
          a.mt_list[3 * n + 1] = r;
          a.mt_list[3 * n + 2] = min(BM, end - r);
          n++;
        }
        lo = end;
      }
    }
    a.mt_off[a.NM] = n;
    // GEMM queue: shared expert, then G1(0), G1(1), G2(0), G1(2), G2(1), ...
    const int nN1 = (2 * a.I + BN - 1) / BN, nN2 = (a.H + BN - 1) / BN;
    const int nN1s = (2 * a.Is + BN - 1) / BN, MTs = (a.T + BM - 1) / BM;
    int p = 0, off = 0;
    auto add = [&](int32_t *kind, int32_t *mm, int32_t *po, int &q, int k_, int m_, int c_) {
      kind[q] = k_; mm[q] = m_; po[q] = off; off += c_; q++;
    };
    if (a.Is > 0) {
      add(a.ph_kind, a.ph_m, a.ph_off, p, PH_SG1, 0, MTs * nN1s);
      add(a.ph_kind, a.ph_m, a.ph_off, p, PH_SG2, 0, MTs * nN2);
    }
    for (int m = 0; m <= a.NM; m++) {
      if (m < a.NM) add(a.ph_kind, a.ph_m, a.ph_off, p, PH_G1, m, (a.mt_off[m + 1] - a.mt_off[m]) * nN1);
      if (m >= 1) add(a.ph_kind, a.ph_m, a.ph_off, p, PH_G2, m - 1, (a.mt_off[m] - a.mt_off[m - 1]) * nN2);
    }
    a.ph_off[p] = off;
    // communication queue: D(0..S-1), then D(m+S), C(m)
    int q = 0;
    off = 0;
    auto dchunks = [&](int m) {
      return (min((m + 1) * a.MB, a.R) - m * a.MB + a.DCH - 1) / a.DCH;
    };
    for (int m = 0; m < min(a.S, a.NM); m++) add(a.cph_kind, a.cph_m, a.cph_off, q, CP_D, m, dchunks(m));
    for (int m = 0; m < a.NM; m++) {
      if (m + a.S < a.NM) add(a.cph_kind, a.cph_m, a.cph_off, q, CP_D, m + a.S, dchunks(m + a.S));
      add(a.cph_kind, a.cph_m, a.cph_off, q, CP_C, m, (cnt[m] + a.CT - 1) / a.CT);
    }
    a.cph_off[q] = off;
  }
  __syncthreads();
  for (int t = tid; t < a.T; t += 256) {
    const int m = a.tok_m[t];
    a.tl[a.tl_off[m] + atomicAdd(&fill[m], 1)] = t;
  }
}

}  // namespace

int launch_layer_fwd_megakernel(const MkArgs &a, int cus, hipStream_t s) {
  // the schedule needs every workgroup resident at once: a cooperative launch
  // guarantees that (or fails), one workgroup per CU
  const void *fn = a.mx ? (const void *)layer_fwd_megakernel<true>
                        : (const void *)layer_fwd_megakernel<false>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0) != hipSuccess ||
      per_cu < 1)
    return -1;
  const int grid = cus;  // one per CU; n_comm < grid is checked by the caller
  hipLaunchKernelGGL(mk_plan_kernel, dim3(1), dim3(256), 0, s, a);
  MkArgs arg = a;
  void *args[] = {&arg};
  if (hipLaunchCooperativeKernel(fn, dim3(grid), dim3(NT), args, 0, s) != hipSuccess) return -1;
  return 0;
}

}  // namespace moe
