// The layer forward as one persistent, pipelined kernel.
//
// The schedule (plan, task queues, waits, signals; mk_schedule.h) runs the
// layer's dispatch, expert GEMM tiles and combine in minibatches inside one
// kernel, with a few workgroups moving rows while the rest run GEMM tiles.
// On one MI355X the "communication" is the HBM gather of dispatch and the
// weighted gather of combine.  The grid is one workgroup per CU (each holds
// the 128 KB of LDS a GEMM tile needs).  The tiles and the combine are the
// staged kernels' own device functions, so the outputs are bit-identical to
// the staged forward.  This file supplies the GPU side of the schedule's two
// interfaces: DevEnv (atomics, polling, fences, barriers, broadcasts through
// LDS) and DevWork (dispatch, combine and GEMM tiles).
#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"
#include "megakernel.h"
#include "row_tile.h"
#include "rows.h"

namespace moe {

static_assert(mk::kStatusOk == MOE_OK && mk::kStatusTimeout == MOE_ERR_DEVICE_TIMEOUT,
              "status codes of the schedule");
static_assert(mk::kTileRows == BM && mk::kTileCols == BN, "schedule tile = GEMM tile");

namespace {

// The GPU side of the schedule's environment.  Polling is a relaxed
// device-scope load on purpose: an acquire load invalidates the XCD's whole
// L2 each time, which starves the producers being waited for; the acquire
// fence is taken once, after the flag is seen (in wait_all).
struct DevEnv {
  mk::Task *sh_task;
  int *sh_fail;
  __device__ int tid() const { return threadIdx.x; }
  __device__ void barrier() const { __syncthreads(); }
  __device__ int atomic_add(int32_t *p, int v) const { return atomicAdd(p, v); }
  __device__ void cas(int32_t *p, int expected, int desired) const {
    atomicCAS(p, expected, desired);
  }
  __device__ int poll(const int32_t *p) const {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ void fence_release() const { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
  __device__ void fence_acquire() const { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
  __device__ void nap(int n) const {
    for (int z = 0; z < n; z++) __builtin_amdgcn_s_sleep(16);  // ~1000 cycles each
  }
  // 100 MHz real-time counter (the watchdog's clock)
  __device__ unsigned long long now() const { return __builtin_amdgcn_s_memrealtime(); }
  __device__ mk::Task bcast(mk::Task t) const {
    if (threadIdx.x == 0) *sh_task = t;
    __syncthreads();
    const mk::Task r = *sh_task;
    __syncthreads();
    return r;
  }
  __device__ int bcast_fail(int f) const {
    if (threadIdx.x == 0) *sh_fail = f;
    __syncthreads();
    const int r = *sh_fail;
    __syncthreads();
    return r;
  }
};

// Shared-memory atomics of the plan kernel.
struct DevPlanOps {
  __device__ static int shared_add(int *p, int v) { return atomicAdd(p, v); }
};

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
  const int HC = a.plan.H / 8;
  const long n = (long)(r1 - r0) * HC;
  for (long id = threadIdx.x; id < n; id += NT) {
    const int r = r0 + (int)(id / HC), c = (int)(id % HC);
    const int src = a.perm[r] / a.plan.k;
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
      if ((c & 3) == 0) a.xs[((size_t)(c >> 4) * a.plan.R + r) * 4 + ((c >> 2) & 3)] = (uint8_t)sc;
      ((uint4 *)a.x_perm)[(size_t)r * HC + c] = pack8(deq);
    }
  }
}

template <bool MX>
struct DevWork {
  const MkArgs &a;
  uint8_t *L0, *L1;
  __device__ void dispatch(int, int r0, int r1) { dispatch_rows<MX>(a, r0, r1); }
  __device__ void combine(int, int b0, int b1) {
    const int HC = a.plan.H / 8;
    for (int id = threadIdx.x; id < (b1 - b0) * HC; id += NT) {
      const int tok = a.plan.tl[b0 + id / HC], c = id % HC;
      combine8(a.y, a.w, a.plan.inv, a.plan.Is > 0 ? a.ys : nullptr, a.out, tok, c, a.plan.k,
               HC);
    }
  }
  __device__ void tile(int kind, int, int, int e, int row0, int rows, int mt, int nt) {
    switch (kind) {
      case mk::PH_SG1:
        run_tile<MX>(a.sg1, a.smx1, EPI_SWIGLU, 0, mt * BM, nt * BN, 0, a.plan.T, L0, L1);
        break;
      case mk::PH_SG2:
        run_tile<MX>(a.sg2, a.smx2, EPI_BF16, 0, mt * BM, nt * BN, 0, a.plan.T, L0, L1);
        break;
      case mk::PH_G1:
        run_tile<MX>(a.g1, a.mx1, EPI_SWIGLU, e, 0, nt * BN, row0, rows, L0, L1);
        break;
      default:
        run_tile<MX>(a.g2, a.mx2, EPI_BF16, e, 0, nt * BN, row0, rows, L0, L1);
        break;
    }
  }
};

template <bool MX>
__global__ __launch_bounds__(NT, 1) void layer_fwd_megakernel(MkArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t L0[2 * BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t L1[2 * BM * 128];
  __shared__ mk::Task sh_task;
  __shared__ int sh_fail;
  DevEnv env{&sh_task, &sh_fail};
  DevWork<MX> work{a, L0, L1};
  mk::run_workgroup(a.plan, (int)blockIdx.x, env, work);
}

// Plan of one call (one workgroup): the schedule's plan phases, separated by
// barriers.
__global__ __launch_bounds__(256) void mk_plan_kernel(MkArgs args) {
  __shared__ int cnt[kMkMaxMinibatches], fill[kMkMaxMinibatches];
  const mk::Plan &a = args.plan;
  const int tid = threadIdx.x;
  mk::plan_zero(a, tid, 256, cnt, fill);
  __syncthreads();
  mk::plan_count<DevPlanOps>(a, tid, 256, cnt);
  __syncthreads();
  if (tid == 0) mk::plan_tables(a, cnt);
  __syncthreads();
  mk::plan_fill<DevPlanOps>(a, tid, 256, fill);
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
