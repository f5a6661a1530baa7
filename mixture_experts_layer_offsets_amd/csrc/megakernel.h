// Arguments of the persistent layer-forward kernel (megakernel.hip).
#pragma once

#include "kernels.h"

namespace moe {

constexpr int kMkMaxMinibatches = 1024;

struct MkArgs {
  // shape and schedule
  int T, H, k, E, I, Is, R, mx;
  int MB, NM, S, n_comm, DCH, CT;
  unsigned long long watchdog_ticks;  // 100 MHz ticks a wait may take
  // layer data
  const uint16_t *x;
  const int32_t *perm, *inv, *offsets;
  const float *w;
  uint16_t *x_perm;        // bf16 rows, or with MXFP8 their round trip
  uint8_t *xq, *xs;        // MXFP8 codes and scales of the rows
  GemmArgs g1, g2, sg1, sg2;  // routed gate/up, down; shared gate/up, down
  MxOperands mx1, mx2, smx1, smx2;
  const uint16_t *y, *ys;
  uint16_t *out;
  // plan (written by the plan kernel)
  int32_t *mt_list;        // [max_tiles][3]: expert, first sorted row, rows
  int32_t *mt_off;         // [NM + 1]
  int32_t *ph_kind, *ph_m, *ph_off;     // GEMM queue phases [n_ph (+1)]
  int32_t *cph_kind, *cph_m, *cph_off;  // communication queue phases [n_cph (+1)]
  int n_ph, n_cph;
  int32_t *tl, *tl_off, *tok_m;         // tokens by last minibatch
  // counters, zeroed by the plan kernel
  int32_t *counters;
  int n_counters;
  int32_t *gemm_next, *comm_next, *disp_done, *g1_done, *g1m_done, *g2m_done, *sg1_done,
      *sg2_done;
  int32_t *status;
};

// Plan kernel + persistent kernel (cooperative launch, one workgroup per CU)
// on stream s; nonzero if the launch was refused.
int launch_layer_fwd_megakernel(const MkArgs &a, int cus, hipStream_t s);

}  // namespace moe
