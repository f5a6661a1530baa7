// Arguments of the persistent layer-forward kernel (megakernel.hip).
#pragma once

#include "kernels.h"
#include "mk_schedule.h"

namespace moe {

constexpr int kMkMaxMinibatches = mk::kMaxMinibatches;

struct MkArgs {
  mk::Plan plan;  // shape, schedule, plan tables and counters
  int mx;
  // layer data
  const uint16_t *x;
  const int32_t *perm;
  const float *w;
  uint16_t *x_perm;        // bf16 rows, or with MXFP8 their round trip
  uint8_t *xq, *xs;        // MXFP8 codes and scales of the rows
  GemmArgs g1, g2, sg1, sg2;  // routed gate/up, down; shared gate/up, down
  MxOperands mx1, mx2, smx1, smx2;
  const uint16_t *y, *ys;
  uint16_t *out;
};

// Plan kernel + persistent kernel (cooperative launch, one workgroup per CU)
// on stream s; nonzero if the launch was refused.
int launch_layer_fwd_megakernel(const MkArgs &a, int cus, hipStream_t s);

}  // namespace moe
