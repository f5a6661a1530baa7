/*
 * moe.h -- C ABI of libmoe: one Mixture-of-Experts layer, forward and
 * backward, on one AMD Instinct MI355X (gfx950).
 *
 * Sources (the pages describe the layer in prose only):
 *   [KC] kucoin.com news flash "O MoK do Cursor alcança aumento de desempenho
 *        de 2,37x no NVIDIA GB300 NVL72", §01 "O imposto sobre comunicações
 *        do MoE", §02 (pull dispatch, megakernel, ring buffer), §03
 *        (benchmark of the whole layer: scheduling, dispatch, the experts'
 *        FFN, combine and the weighted sum that ends it).
 *   [NA] noticiai.com.br "Cursor abre código do Mixture-of-Kittens: kernel
 *        MoE que acelera treinamento em GPUs Blackwell em até 2,37×",
 *        section "As três decisões de design que fazem a diferença".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device buffers must be device memory of the current
 *   HIP device; all other pointers (shapes, schedules, status) are host.
 * - bf16 tensors are passed as uint16_t bit patterns, row-major.
 * - Shapes: T tokens, H hidden, E routed experts, k top-k, I expert
 *   intermediate size, R = T*k routed rows, Is shared-expert intermediate.
 *   Expert weights are row-major with the layer computing x*W:
 *   w_gate, w_up [E][H][I]; w_down [E][I][H]; router [H][E].
 * - Rows: f = t*k + j is the flat (token, slot) index; r is the row in
 *   expert-sorted order.  perm[r] = f and inv_perm[f] = r.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every call only enqueues work on it and returns; no call waits for the
 *   device (the only exception is moe_read_status).  Inputs must stay
 *   unchanged and outputs unread until the stream has passed the call.
 * - The library allocates no device memory and keeps no state between
 *   calls: scratch comes from the caller's workspace (`ws`, `ws_bytes`,
 *   sized by moe_workspace_bytes) and the forward->backward context from
 *   the caller's `saved` buffer (moe_saved_bytes).  Calls on one stream with
 *   distinct workspaces may be issued from several threads.
 * - Results are deterministic: the same inputs give bitwise-identical
 *   outputs, run to run (no floating-point atomics; every reduction has a
 *   fixed order).
 * - No token is dropped and no buffer depends on the routing: every (t, j)
 *   owns one row (the pages' ring buffer exists so that neither tokens are
 *   dropped nor the CPU sizes buffers per step [NA design, item 3]).
 * - Errors: each int-returning call returns MOE_OK or one of the codes
 *   below and enqueues nothing when it fails its argument checks.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* NULL required pointer, size <= 0, k > E when routing, overflow */
  MOE_ERR_UNSUPPORTED = 2,   /* shape outside the kernels' limits (see moe_shape) */
  MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4,           /* a HIP launch or copy failed */
  MOE_ERR_DEVICE_TIMEOUT = 5 /* reported by moe_read_status only */
};

/* Datatypes of the layer.
 * MOE_BF16: bf16 activations and weights, fp32 accumulation.
 * MOE_MXFP8: every operand of the expert GEMMs in MXFP8 (E4M3 codes, one
 *   E8M0 scale per 32 values along the contraction axis), quantised in the
 *   dispatch and the SwiGLU epilogue [KC §02]; weights pre-quantised.
 * MOE_MXFP8_W4, MOE_MXFP8_W6, MOE_MXFP8_W6E3M2: lower-precision experts --
 *   the expert weights' MX copies in FP4 E2M1, FP6 E2M3 or FP6 E3M2 (one
 *   E8M0 scale per 32 values, OCP MX conversion: nearest-even, saturating at
 *   the format's maximum), the activations and gradients MXFP8 as above; the
 *   pages mention 4-bit expert kernels (noticiai.com.br, "Por que a camada
 *   MoE virou o gargalo").  FP4 weights take half the bytes of FP8 ones; FP6
 *   blocks are stored in 32-byte slots (24 bytes of codes), so FP6 weights
 *   take the bytes of FP8 ones. */
enum {
  MOE_BF16 = 0,
  MOE_MXFP8 = 1,
  MOE_MXFP8_W4 = 2,
  MOE_MXFP8_W6 = 3,
  MOE_MXFP8_W6E3M2 = 4
};

/* The layer's shape, following the quantities the pages tune the layer by:
 * hidden size, top-k and expert count [KC §03], expert intermediate size
 * [KC §02], plus the token count and the datatype.
 * Limits: 1 <= T; 1 <= k <= 16; 1 <= E <= 1024; H, I and shared_inter
 * multiples of 64 (of 128 for the MX types); R = T*k < 2^31; H*E < 2^31.
 * The MX types also: with Rp = R + 127 E rounded up to a multiple of 128
 * (the routed rows padded per expert), Rp < 2^23, Rp * max(H, 2 I,
 * 2 shared_inter) < 2^36 and E * H * max(I, shared_inter) < 2^35 (32-bit
 * byte counts of the scaled operands).  Other shapes: MOE_ERR_UNSUPPORTED. */
typedef struct moe_shape {
  int32_t tokens;       /* T */
  int32_t hidden;       /* H */
  int32_t experts;      /* E: routed experts held by this GPU */
  int32_t top_k;        /* k */
  int32_t inter;        /* I */
  int32_t shared_inter; /* Is of the one shared expert; 0 = no shared expert */
  int32_t dtype;        /* MOE_BF16, MOE_MXFP8 or a lower-precision-expert type */
} moe_shape;

/* How the layer's forward and backward are scheduled (moe_sched.schedule).
 *
 * MOE_SCHED_STAGED: one kernel per step over all rows, on the caller's
 *   stream.
 * MOE_SCHED_PERSISTENT: the forward as one persistent kernel with a CU split
 *   and device flags.  Switched off: refused with MOE_ERR_UNSUPPORTED.
 * MOE_SCHED_PIPELINED: the rows go through the experts in minibatches
 *   [KC §02]: minibatch m's dispatch overlaps the GEMMs of earlier
 *   minibatches, and each token is combined as soon as the minibatch holding
 *   its last routed row is done.  Dispatch, combine and their backward
 *   mirrors run on a communication stream; the GEMMs of even and odd
 *   minibatches run on two GEMM streams, so one minibatch's GEMMs can fill the
 *   compute units the previous one leaves idle.  All ordering is by HIP events
 *   on the GPU, with no host wait per minibatch [KC §02].  The backward walks
 *   the minibatches in reverse [NA design].  With comm_cus > 0 the
 *   communication stream is limited to comm_cus CUs and the GEMM streams to
 *   the rest (hardware CU masks); with comm_cus = 0 all three share every CU.
 *   The streams and events are the library's own: one set of three streams
 *   per comm_cus value, created on the first pipelined call with that value
 *   on each device and kept until the process ends, so no call waits for
 *   earlier work; at most 8 distinct comm_cus values per device (a ninth is
 *   refused with MOE_ERR_UNSUPPORTED, and comm_cus >= the device's CU count
 *   with MOE_ERR_INVALID_ARG, before anything is enqueued).  Pipelined calls
 *   on one device are enqueued one at a time (a mutex); every call forks
 *   from and joins back to the caller's stream, so calls on one caller
 *   stream execute in call order.  Outputs are bit-identical to
 *   MOE_SCHED_STAGED. */
enum { MOE_SCHED_STAGED = 0, MOE_SCHED_PERSISTENT = 1, MOE_SCHED_PIPELINED = 2 };

/* Schedule knobs of the layer call.  The pages retune the minibatch and the
 * number of communication processors per model shape [KC §03]; 0 always
 * means "library default".
 *
 * stage_events (optional, host array of caller-created hipEvent_t, cast to
 * void*): when non-NULL the layer calls record event i on `stream` at stage
 * boundary i, for i < n_stage_events, so a caller can time each stage:
 *   forward : 0 start, 1 routing+layout done, 2 dispatch done, 3 gate/up
 *             GEMM + SwiGLU done, 4 down GEMM done, 5 shared expert done,
 *             6 combine done (pipelined: 2-6 are recorded when all streams
 *             have joined the caller's stream again);
 *   backward: 0 start, 1 reverse-combine done, 2 down data-gradient GEMM
 *             (+ SwiGLU backward) done, 3 down weight-gradient GEMM done,
 *             4 gate/up data-gradient GEMM done, 5 gate/up weight-gradient
 *             GEMM done, 6 shared expert done, 7 router + reverse-dispatch
 *             done (pipelined: 1-7 at the join). */
typedef struct moe_sched {
  int32_t minibatch_rows; /* routed rows per minibatch (0 = default: enough
                             rows for two full waves of 256 x 256 tiles of
                             the direction's first GEMM -- gate/up forward,
                             down data gradient backward -- and in the
                             forward at least half the rows; always at
                             least max(256, ceil(R / 1024))).  A
                             one-minibatch pipelined forward is the staged
                             forward, on the caller's stream. */
  int32_t ring_slots;     /* minibatches dispatched ahead of the gate/up GEMM
                             (0 = default, 2) */
  int32_t comm_cus;       /* CUs given to dispatch/combine (0 = share all) */
  int32_t schedule;       /* MOE_SCHED_* (0 = staged) */
  void **stage_events;    /* hipEvent_t[n_stage_events] or NULL */
  int32_t n_stage_events;
  int32_t watchdog_us;    /* persistent kernel only: microseconds one wait may
                             take before it gives up (0 = default, 2 s) */
  int32_t mx_wgrad;       /* MXFP8 shapes: 1 = the weight-gradient GEMMs also
                             take MX operands, quantised down the rows (the
                             GEMMs' contraction axis) in E8M0 blocks of 32
                             rows starting at each expert's first row, the
                             last block zero-padded; 0 (default) = bf16
                             weight gradients on the MX round trips */
  void (*stage_hook)(void *user, int32_t stage);
                          /* optional, with stage_events: called on the
                             calling thread while the layer call enqueues,
                             just before boundary `stage` (< n_stage_events)
                             is recorded, so a caller can enqueue work of
                             its own on `stream` ahead of that stage (a
                             benchmark's cache flush); NULL = none */
  void *stage_hook_user;  /* passed to stage_hook */
  uint64_t *kernel_stamps;
                          /* optional device array of 8 * n_stage_events
                             words, zeroed by the caller, staged schedule
                             only: every tile of the expert GEMMs enqueued in
                             stage i (the work after boundary i) adds, with
                             device atomics, to words 8i + 0..4: tiles,
                             shader cycles from tile start to epilogue end,
                             of which the prologue and K loop, and the
                             epilogue, and real-time ticks (100 MHz) -- so
                             cycles / ticks * 100 MHz is the clock the tiles
                             ran at.  Read it after the stream is done.
                             NULL = no timing (the default) */
} moe_sched;

/* ------------------------------------------------------------------ sizes */

/* Bytes of scratch every call below needs at most for this shape (host call,
 * no device work).  Depends only on the shape, never on the routing. */
size_t moe_workspace_bytes(const moe_shape *shape);

/* Bytes of the forward->backward context written by moe_layer_fwd. */
size_t moe_saved_bytes(const moe_shape *shape);

/* Bytes of the packed weights written by moe_prepare_weights. */
size_t moe_packed_weight_bytes(const moe_shape *shape);

/* ---------------------------------------------------------------- weights */

/* Repack the expert weights into the layouts the grouped GEMMs read (the
 * grouped GEMM wants expert-ordered, contraction-contiguous operands
 * [KC §01]).  Inputs (device, bf16): w_gate, w_up [E][H][I], w_down
 * [E][I][H]; the shared expert's ws_gate, ws_up [H][Is], ws_down [Is][H]
 * (all three NULL when shared_inter == 0).  Output: `packed` (device,
 * moe_packed_weight_bytes, caller-owned, opaque).  With MXFP8 the packed
 * buffer also holds E4M3+E8M0 copies quantised along each GEMM's
 * contraction axis.  Call again whenever the weights change. */
int moe_prepare_weights(const moe_shape *shape, const uint16_t *w_gate,
                        const uint16_t *w_up, const uint16_t *w_down,
                        const uint16_t *ws_gate, const uint16_t *ws_up,
                        const uint16_t *ws_down, void *packed, void *stream);

/* ------------------------------------------------------------- the steps */

/* Router logits: logits[t][e] = fp32(sum_h x[t][h] * w_router[h][e]) +
 * bias[e] (bias may be NULL).  The router re-decides every step which
 * experts a token visits [KC §01].  x [T][H] bf16, w_router [H][E] bf16,
 * logits [T][E] fp32 (all device).  E must be a multiple of 8 (whole 16-byte
 * rows of w_router); other E return MOE_ERR_UNSUPPORTED. */
int moe_router_logits(const moe_shape *shape, const uint16_t *x,
                      const uint16_t *w_router, const float *bias,
                      float *logits, void *ws, size_t ws_bytes, void *stream);

/* Top-k selection and weights: per token, the k largest logits (equal
 * logits: lower expert index first), slot j = j-th largest; weights =
 * softmax over the k selected logits, in fp32.  Each token picks a few
 * experts [KC §01].  logits [T][E] fp32 -> topk_idx [T][k] int32,
 * topk_w [T][k] fp32.  Requires k <= E. */
int moe_route(const moe_shape *shape, const float *logits, int32_t *topk_idx,
              float *topk_w, void *stream);

/* Layout ("Schedule"): count rows per expert, prefix-sum them, and order
 * rows expert-contiguously, stable in f [KC §01].  topk_idx [T][k] int32
 * (every entry in [0, E); duplicates within a token allowed) ->
 * counts [E], offsets [E+1], perm [R], inv_perm [R] (int32, device).
 * Bit-exact and deterministic.  Entries outside [0, E) are not checked on
 * the host; the kernels clamp them into [0, E) and the result is then
 * undefined but memory-safe. */
int moe_layout(const moe_shape *shape, const int32_t *topk_idx,
               int32_t *counts, int32_t *offsets, int32_t *perm,
               int32_t *inv_perm, void *ws, size_t ws_bytes, void *stream);

/* Layout without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same results as moe_layout, bit for bit, with its
 * scratch (per-chunk expert counts, tile prefix, expert order) in a static
 * device array of the library, 4 MiB per device, held until the process
 * ends.  Shapes whose scratch exceeds it -- ceil(T*k / 1024) * E + 2E + 1
 * int32 words, each of the three pieces rounded up to 256 bytes -- return
 * MOE_ERR_WORKSPACE and enqueue nothing.  The call allocates nothing and
 * does not wait for the device.  Every call on one device shares that
 * device's array: calls whose work overlaps on the device (different
 * streams, or several threads) race and give undefined results; calls
 * ordered on one stream are safe.  Arguments and errors otherwise as
 * moe_layout. */
int moe_layout_noalloc(const moe_shape *shape, const int32_t *topk_idx,
                       int32_t *counts, int32_t *offsets, int32_t *perm,
                       int32_t *inv_perm, void *stream);

/* Dispatch (gather-permute): row r of x_perm is a copy of token
 * perm[r] / k of x -- the destination-driven read the pages call pull
 * dispatch [KC §02].  bf16: x_perm is uint16_t [R][H], x_scale unused.
 * MXFP8: x_perm is E4M3 codes uint8 [R][H] and x_scale the E8M0 scales,
 * one per 32 values along H, quantised as the row is copied [KC §02].
 * MX scale layout (x_scale here and every E8M0 array below): K-blocked,
 * [K/128][rows][4] -- the scale of row r and 32-block b of a [rows][K]
 * matrix is byte (b/4 * rows + r) * 4 + b%4, so the scales of one 128-wide
 * K slice of consecutive rows are consecutive dwords (what a GEMM tile
 * reads per stage).  rows = R here. */
int moe_dispatch(const moe_shape *shape, const uint16_t *x,
                 const int32_t *perm, void *x_perm, uint8_t *x_scale,
                 void *stream);

/* Expert FFN as grouped GEMMs over the expert-contiguous rows [KC §01]:
 * for the rows [offsets[e], offsets[e+1]) of expert e,
 * a = silu(X w_gate[e]) * (X w_up[e]) (SwiGLU fused in the GEMM epilogue),
 * y = a w_down[e].  x_perm/x_scale as written by moe_dispatch, offsets
 * [E+1], packed from moe_prepare_weights, y [R][H] bf16 (device).  The
 * intermediate activations live in the workspace.  MXFP8: the gate/up GEMM
 * reads E4M3 codes with their E8M0 scales, the SwiGLU epilogue quantises a
 * along I (32-wide blocks) and the down GEMM reads those codes [KC §02]. */
int moe_expert_ffn(const moe_shape *shape, const void *x_perm,
                   const uint8_t *x_scale, const int32_t *offsets,
                   const void *packed, uint16_t *y, void *ws, size_t ws_bytes,
                   void *stream);

/* Combine and final weighted fusion [KC §03]: out[t] = bf16( sum_{j<k}
 * topk_w[t][j] * y[inv_perm[t*k+j]] + y_shared[t] ), fp32 accumulation in
 * ascending j.  y [R][H], y_shared [T][H] (may be NULL), out [T][H] bf16. */
int moe_combine(const moe_shape *shape, const uint16_t *y,
                const float *topk_w, const int32_t *inv_perm,
                const uint16_t *y_shared, uint16_t *out, void *stream);

/* ------------------------------------------------------------- the layer */

/* Whole forward, the layer the pages measure end to end [KC §03]:
 * scheduling ([router logits, top-k] or supplied routing, then layout),
 * dispatch, the expert FFN (+ the shared expert), combine and the final
 * weighted sum.
 * Routing: pass w_router (+ optional bias) with topk_idx_in = topk_w_in =
 * NULL (then k <= E, and E a multiple of 8 as for moe_router_logits), or
 * pass topk_idx_in [T][k] / topk_w_in [T][k] (device) with
 * w_router = NULL (any E).  x [T][H] bf16, out [T][H] bf16, saved (device,
 * moe_saved_bytes) receives the context moe_layer_bwd reads.  `sched` may
 * be NULL (defaults). */
int moe_layer_fwd(const moe_shape *shape, const moe_sched *sched,
                  const uint16_t *x, const uint16_t *w_router,
                  const float *bias, const int32_t *topk_idx_in,
                  const float *topk_w_in, const void *packed, uint16_t *out,
                  void *saved, void *ws, size_t ws_bytes, void *stream);

/* Whole backward, mirroring the forward's data movement [KC §01, §02]:
 * reverse-combine, SwiGLU expert backward (data and weight gradients),
 * reverse-dispatch, router backward.  dout [T][H] bf16; x and w_router as
 * given to the forward (w_router NULL for supplied routing); saved from
 * moe_layer_fwd.  Outputs (device): dx [T][H] bf16; dw_gate, dw_up
 * [E][H][I] fp32; dw_down [E][I][H] fp32; dw_router [H][E] fp32 (router
 * routing, else NULL); dws [H*Is | H*Is | Is*H] fp32 = shared expert's
 * d(gate), d(up), d(down) (NULL without a shared expert); dtopk_w [T][k]
 * fp32 = gradient of the routing weights (may be NULL).  Every output is
 * fully written (experts that received no rows get zero gradients).
 * MXFP8: the two data-gradient GEMMs read MX copies of dY (along H) and of
 * dg|du (along I) against weights quantised along the same axes; the weight
 * gradients are bf16 products of the forward's MX round trips and the bf16
 * gradients. */
int moe_layer_bwd(const moe_shape *shape, const moe_sched *sched,
                  const uint16_t *dout, const uint16_t *x,
                  const uint16_t *w_router, const void *saved,
                  const void *packed, uint16_t *dx, float *dw_router,
                  float *dw_gate, float *dw_up, float *dw_down, float *dws,
                  float *dtopk_w, void *ws, size_t ws_bytes, void *stream);

/* Few-token inference forward (decode): the same layer output as
 * moe_layer_fwd -- routing, layout, expert FFN, shared expert, combine --
 * for a small token count, with no forward context and no backward.  The
 * pages mention a separate decode kernel for inference in which each token
 * gets its own small group of threads [NA design].  With few tokens the
 * layer is bound by reading the selected experts' weights, so the expert FFN
 * here streams each used expert's packed weight rows once per pass, a deep
 * ring of them in flight per wave, and applies them on the matrix cores to
 * all of that expert's routed rows (64 per pass; an expert with more rows
 * re-reads its weights per 64), with fp32 accumulation in a fixed order
 * (deterministic).  Meant for T*k up to a few hundred rows; larger batches
 * belong to moe_layer_fwd's MFMA grouped GEMMs.  Arguments as moe_layer_fwd (x [T][H]
 * bf16; router w_router/bias or supplied topk_idx/topk_w; packed from
 * moe_prepare_weights; out [T][H] bf16; ws of moe_workspace_bytes).  bf16
 * only: MXFP8 shapes return MOE_ERR_UNSUPPORTED. */
int moe_decode_fwd(const moe_shape *shape, const uint16_t *x,
                   const uint16_t *w_router, const float *bias,
                   const int32_t *topk_idx_in, const float *topk_w_in,
                   const void *packed, uint16_t *out, void *ws,
                   size_t ws_bytes, void *stream);

/* Device pointers into a forward context (host call, no device work):
 * where moe_layer_fwd left each intermediate.  Any field may be NULL in
 * the result when the shape has no such tensor. */
typedef struct moe_saved_view {
  int32_t *topk_idx;  /* [T][k] */
  float *topk_w;      /* [T][k] */
  float *logits;      /* [T][E] (router routing) */
  int32_t *counts;    /* [E] */
  int32_t *offsets;   /* [E+1] */
  int32_t *perm;      /* [R] */
  int32_t *inv_perm;  /* [R] */
  void *x_perm;       /* bf16 [R][H] (bf16), or E4M3 codes [R][H] (MXFP8) */
  uint8_t *x_scale;   /* E8M0, K-blocked [H/128][R][4] (MXFP8) */
  uint16_t *x_hat;    /* bf16 [R][H]: MX round trip of the dispatched rows (MXFP8) */
  uint16_t *gu;       /* bf16 [R][2I]: g and u, interleaved in 32-column blocks */
  uint16_t *act;      /* bf16 [R][I]: a (bf16) or its MX round trip (MXFP8) */
  uint8_t *act_q;     /* E4M3 [R][I] (MXFP8) */
  uint8_t *act_scale; /* E8M0, K-blocked [I/128][R][4] (MXFP8) */
  uint16_t *y;        /* bf16 [R][H] */
  uint16_t *y_shared; /* bf16 [T][H] (shared expert) */
} moe_saved_view;

int moe_saved_pointers(const moe_shape *shape, void *saved,
                       moe_saved_view *view);

/* Device pointers into packed weights (host call, no device work): where
 * moe_prepare_weights left the routed experts' MX copies (NULL for
 * MOE_BF16).  Each copy is the weights laid out contraction-contiguous for
 * one GEMM and quantised along that contraction axis, with E8M0 scales in
 * the K-blocked layout of moe_dispatch:
 *   gate_up  [E][2I][H]: gate and up interleaved in 32-row blocks (rows
 *            64b .. 64b+31 = gate columns 32b .. 32b+31, the next 32 = up
 *            columns), quantised along H (the forward gate/up GEMM);
 *   down     [E][H][I] quantised along I (the forward down GEMM);
 *   gate_up_t [E][H][2I] (the same interleave along 2I), quantised along 2I
 *            (the gate/up data-gradient GEMM);
 *   down_t   [E][I][H] quantised along H (the down data-gradient GEMM).
 * Codes: one byte per value for E4M3; for FP6 each 32-value block takes 32
 * bytes (24 bytes of 6-bit codes, value p at bits 6p.., then 8 zero bytes);
 * for FP4 16 bytes (value p at bits 4p..), rows of half the values' count.
 * fmt is the dtype's weight format: 0 E4M3, 2 FP6 E2M3, 3 FP6 E3M2,
 * 4 FP4 E2M1. */
typedef struct moe_packed_view {
  uint8_t *gate_up;
  uint8_t *gate_up_scale;
  uint8_t *down;
  uint8_t *down_scale;
  uint8_t *gate_up_t;
  uint8_t *gate_up_t_scale;
  uint8_t *down_t;
  uint8_t *down_t_scale;
  int32_t fmt;
} moe_packed_view;

int moe_packed_pointers(const moe_shape *shape, void *packed, moe_packed_view *view);

/* Device pointers into a workspace (host call, no device work): where the
 * last call that used `ws` left its intermediates, for callers that inspect
 * them (valid until the next call that uses `ws`).  Fields are NULL when
 * the shape is invalid. */
typedef struct moe_work_view {
  uint16_t *dy;       /* moe_layer_bwd: bf16 [R][H], rows' output gradient
                         (reverse-combine) */
  uint16_t *dh;       /* moe_layer_bwd: bf16 [R][2I], dg and du interleaved in
                         32-column blocks */
  uint16_t *dx_rows;  /* moe_layer_bwd: bf16 [R][H], rows' input gradient
                         (before reverse-dispatch) */
  float *dec_logits;  /* moe_decode_fwd with a router: fp32 [T][E] logits */
  int32_t *dec_topk_idx; /* moe_decode_fwd with a router: [T][k] selection */
  float *dec_topk_w;  /* moe_decode_fwd with a router: fp32 [T][k] weights
                         (with supplied routing the decode reads the caller's
                         arrays in place and writes none of these three) */
  /* moe_layer_bwd with MXFP8 (NULL in bf16): the data-gradient GEMMs' MX
     operands, each the row quantisation of the bf16 tensor above (E8M0
     scale per 32 consecutive values of a row, [KC §02] MXFP8 backward).
     Codes are E4M3 bytes, row-major like the bf16 tensor; scales are
     K-blocked, block b of row r at byte (b/4 * R + r) * 4 + b%4. */
  uint8_t *dy_codes;  /* [R][H], written by the reverse-combine */
  uint8_t *dy_scales; /* [H/128][R][4] */
  uint8_t *dh_codes;  /* [R][2I] */
  uint8_t *dh_scales; /* [2I/128][R][4] */
} moe_work_view;

int moe_workspace_pointers(const moe_shape *shape, void *ws, moe_work_view *view);

/* Reads the device status word of the last layer call that used `ws`
 * (synchronises `stream`).  *status_host = MOE_OK or MOE_ERR_DEVICE_TIMEOUT. */
int moe_read_status(const void *ws, int32_t *status_host, void *stream);

/* Static description of an error code. */
const char *moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
