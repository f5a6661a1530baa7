// Schedule of the persistent layer forward: the plan, the two task queues,
// their waits and signals.  Written once, against two small interfaces, so
// that the GPU kernel (megakernel.hip) and a host model (one thread per
// workgroup, used by the tests) run the same code:
//
//   Env   tid(), barrier(), atomic_add(p, v) (device scope, returns the old
//         value), cas(p, expected, desired), poll(p) (device-scope relaxed
//         load), fence_release(), fence_acquire(), nap(n), now() (100 MHz
//         ticks), bcast(Task) (thread 0's value to every thread of the
//         workgroup), bcast_fail(int);
//   Work  dispatch(m, r0, r1), combine(m, b0, b1), tile(kind, m, idx, e,
//         row0, rows, mt, nt) -- the data-parallel bodies.
//
// The pages overlap the layer's communication with its expert GEMMs inside
// one kernel: a few processors move rows while the rest run GEMM tiles, the
// routed rows flow in minibatches through a bounded on-device buffer, and
// completion is signalled by flags rather than by the host (kucoin.com news
// flash "O MoK do Cursor alcança aumento de desempenho de 2,37x no NVIDIA
// GB300 NVL72", sections 01-03; deepdigest.ru article on MoK).
//
// Sorted routed rows are cut into minibatches of MB rows; per minibatch m:
//   D(m)  dispatch of its rows, in chunks of DCH rows;
//   G1(m) gate/up + SwiGLU tiles of its rows (wait for all of D(m));
//   G2(m) down tiles (wait for every G1 tile of the same row tile);
//   C(m)  combine of the tokens whose last routed row lies in minibatch m,
//         CT tokens per task (wait for G2 of every minibatch up to m, and the
//         shared expert).
// Communication queue: D(0..S-1), then D(m+S), C(m) for m = 0, 1, ...; D(m)
// for m >= S waits until G1(m-S) is complete (at most S minibatches between
// dispatch and the GEMMs: the pages' S-slot ring as an in-flight window).
// GEMM queue: the shared expert's gate/up tiles, its down tiles (each waits
// for the gate/up tiles of its row tile), then G1(0), G1(1), G2(0), G1(2),
// G2(1), ...  Both queues hand out tasks through an atomic counter, and each
// task waits only for tasks earlier in one of the two orders.
//
// Every wait is bounded: a wait that outlasts watchdog_ticks, or that sees
// another workgroup's failure in the status word, fails and leaves
// MOE_ERR_DEVICE_TIMEOUT there; the workgroup then returns.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

namespace moe {
namespace mk {

constexpr int kMaxMinibatches = 1024;
constexpr int kTileRows = 256, kTileCols = 256;  // the GEMM tile
constexpr int kStatusOk = 0, kStatusTimeout = 5;  // MOE_OK, MOE_ERR_DEVICE_TIMEOUT

enum { PH_SG1 = 0, PH_SG2 = 1, PH_G1 = 2, PH_G2 = 3 };
enum { CP_D = 0, CP_C = 1 };

// What the schedule reads and writes (device pointers on the GPU).
struct Plan {
  int T, H, k, E, I, Is, R;
  int MB, NM, S, n_comm, DCH, CT;
  unsigned long long watchdog_ticks;  // 100 MHz ticks a wait may take
  const int32_t *inv, *offsets;       // layout: row of (t, j); expert row ranges
  int32_t *mt_list;                   // [max_tiles][3]: expert, first sorted row, rows
  int32_t *mt_off;                    // [NM + 1]: first row tile of each minibatch
  int32_t *ph_kind, *ph_m, *ph_off;     // GEMM queue phases [n_ph (+1)]
  int32_t *cph_kind, *cph_m, *cph_off;  // communication queue phases [n_cph (+1)]
  int n_ph, n_cph;
  int32_t *tl, *tl_off, *tok_m;  // tokens grouped by the minibatch of their last row
  int32_t *counters;             // every counter below, zeroed by the plan
  int n_counters;
  int32_t *gemm_next, *comm_next, *disp_done, *g1_done, *g1m_done, *g2m_done, *sg1_done,
      *sg2_done;
  int32_t *status;
};

struct Task {
  int kind, m, local, ok;
};

MK_HD inline int imin(int a, int b) { return a < b ? a : b; }
MK_HD inline int imax(int a, int b) { return a > b ? a : b; }

// Column tiles of the gate/up GEMM (routed, shared) and of the down GEMM.
MK_HD inline int n_cols1(const Plan &a) { return (2 * a.I + kTileCols - 1) / kTileCols; }
MK_HD inline int n_cols1s(const Plan &a) { return (2 * a.Is + kTileCols - 1) / kTileCols; }
MK_HD inline int n_cols2(const Plan &a) { return (a.H + kTileCols - 1) / kTileCols; }
MK_HD inline int shared_row_tiles(const Plan &a) { return (a.T + kTileRows - 1) / kTileRows; }
// Dispatch chunks of minibatch m.
MK_HD inline int dispatch_chunks(const Plan &a, int m) {
  return (imin((m + 1) * a.MB, a.R) - m * a.MB + a.DCH - 1) / a.DCH;
}

// ---- sizes of the plan's arrays, and binding them to memory

// Smallest minibatch the schedule accepts (so that at most kMaxMinibatches
// exist), and the resulting bound on the minibatch count.
MK_HD inline long min_minibatch(long R) {
  const long m = (R + kMaxMinibatches - 1) / kMaxMinibatches;
  return m > 256 ? m : 256;
}
MK_HD inline int max_minibatches(long R) {
  const long mb = min_minibatch(R);
  return (int)((R + mb - 1) / mb);
}
// Bound on the row tiles of any cut: every segment (a minibatch's rows of
// one expert) adds at most one partly filled tile, and there are at most
// E + NM - 1 segments.
MK_HD inline int max_row_tiles(long R, long E, int max_nm) {
  return (int)((R + kTileRows - 1) / kTileRows + E + max_nm + 1);
}
MK_HD inline int counter_words(long T, int max_nm, int max_tiles) {
  return 2 + 3 * max_nm + max_tiles + (int)((T + kTileRows - 1) / kTileRows) + 1;
}
// Words of each table: mt_list, mt_off, ph, cph, tl_off (tl and tok_m take T).
MK_HD inline long mt_list_words(int max_tiles) { return 3L * max_tiles; }
MK_HD inline long ph_words(int max_nm) { return 3L * (2 * max_nm + 3); }
MK_HD inline long cph_words(int max_nm) { return 3L * (2 * max_nm + 1); }

// Points the plan's tables and counters into caller-provided arrays of the
// sizes above (ph holds kind, minibatch and prefix planes of 2 max_nm + 3
// entries; cph the same with 2 max_nm + 1; counters counter_words words).
MK_HD inline void bind(Plan &pl, int max_nm, int max_tiles, int32_t *mt_list, int32_t *mt_off,
                       int32_t *ph, int32_t *cph, int32_t *tl, int32_t *tl_off, int32_t *tok_m,
                       int32_t *counters, int32_t *status) {
  pl.mt_list = mt_list;
  pl.mt_off = mt_off;
  const int nph = 2 * max_nm + 3, ncph = 2 * max_nm + 1;
  pl.ph_kind = ph;
  pl.ph_m = ph + nph;
  pl.ph_off = ph + 2 * nph;
  pl.cph_kind = cph;
  pl.cph_m = cph + ncph;
  pl.cph_off = cph + 2 * ncph;
  pl.n_ph = 2 * pl.NM + (pl.Is > 0 ? 2 : 0);
  pl.n_cph = 2 * pl.NM;
  pl.tl = tl;
  pl.tl_off = tl_off;
  pl.tok_m = tok_m;
  pl.counters = counters;
  pl.n_counters = counter_words(pl.T, max_nm, max_tiles);
  pl.gemm_next = counters;
  pl.comm_next = counters + 1;
  pl.disp_done = counters + 2;
  pl.g1m_done = pl.disp_done + max_nm;
  pl.g2m_done = pl.g1m_done + max_nm;
  pl.g1_done = pl.g2m_done + max_nm;
  pl.sg1_done = pl.g1_done + max_tiles;
  pl.sg2_done = pl.sg1_done + (pl.T + kTileRows - 1) / kTileRows;
  pl.status = status;
}

// ---- the plan (one workgroup of nthr threads; phases separated by barriers)

// Phase 0, every thread: zero the counters and the per-minibatch counts.
MK_HD inline void plan_zero(const Plan &a, int tid, int nthr, int *cnt, int *fill) {
  for (int i = tid; i < a.n_counters; i += nthr) a.counters[i] = 0;
  for (int m = tid; m < a.NM; m += nthr) {
    cnt[m] = 0;
    fill[m] = 0;
  }
}

// Phase 1, every thread: the minibatch of each token's last routed row
// (Ops::shared_add is an atomic add on workgroup-shared memory).
template <class Ops>
MK_HD void plan_count(const Plan &a, int tid, int nthr, int *cnt) {
  for (int t = tid; t < a.T; t += nthr) {
    int last = 0;
    for (int j = 0; j < a.k; j++) last = imax(last, a.inv[t * a.k + j]);
    const int m = last / a.MB;
    a.tok_m[t] = m;
    Ops::shared_add(&cnt[m], 1);
  }
}

// Phase 2, one thread: token-list offsets, the row tiles of every minibatch
// (cut at expert boundaries, 256 rows per tile) and both queues' phase
// tables.
MK_HD inline void plan_tables(const Plan &a, const int *cnt) {
  int s = 0;
  for (int m = 0; m < a.NM; m++) {
    a.tl_off[m] = s;
    s += cnt[m];
  }
  a.tl_off[a.NM] = s;
  int n = 0, e = 0;
  for (int m = 0; m < a.NM; m++) {
    a.mt_off[m] = n;
    int lo = m * a.MB;
    const int hi = imin(a.R, lo + a.MB);
    while (lo < hi) {
      while (a.offsets[e + 1] <= lo) e++;
      const int end = imin(hi, a.offsets[e + 1]);
      for (int r = lo; r < end; r += kTileRows) {
        a.mt_list[3 * n] = e;
        a.mt_list[3 * n + 1] = r;
        a.mt_list[3 * n + 2] = imin(kTileRows, end - r);
        n++;
      }
      lo = end;
    }
  }
  a.mt_off[a.NM] = n;
  const int nN1 = n_cols1(a), nN2 = n_cols2(a), nN1s = n_cols1s(a), MTs = shared_row_tiles(a);
  // GEMM queue: shared expert, then G1(0), G1(1), G2(0), G1(2), G2(1), ...
  int p = 0, off = 0;
  auto add = [&](int32_t *kind, int32_t *mm, int32_t *po, int &q, int k_, int m_, int c_) {
    kind[q] = k_;
    mm[q] = m_;
    po[q] = off;
    off += c_;
    q++;
  };
  if (a.Is > 0) {
    add(a.ph_kind, a.ph_m, a.ph_off, p, PH_SG1, 0, MTs * nN1s);
    add(a.ph_kind, a.ph_m, a.ph_off, p, PH_SG2, 0, MTs * nN2);
  }
  for (int m = 0; m <= a.NM; m++) {
    if (m < a.NM)
      add(a.ph_kind, a.ph_m, a.ph_off, p, PH_G1, m, (a.mt_off[m + 1] - a.mt_off[m]) * nN1);
    if (m >= 1)
      add(a.ph_kind, a.ph_m, a.ph_off, p, PH_G2, m - 1, (a.mt_off[m] - a.mt_off[m - 1]) * nN2);
  }
  a.ph_off[p] = off;
  // communication queue: D(0..S-1), then D(m+S), C(m)
  int q = 0;
  off = 0;
  for (int m = 0; m < imin(a.S, a.NM); m++)
    add(a.cph_kind, a.cph_m, a.cph_off, q, CP_D, m, dispatch_chunks(a, m));
  for (int m = 0; m < a.NM; m++) {
    if (m + a.S < a.NM)
      add(a.cph_kind, a.cph_m, a.cph_off, q, CP_D, m + a.S, dispatch_chunks(a, m + a.S));
    add(a.cph_kind, a.cph_m, a.cph_off, q, CP_C, m, (cnt[m] + a.CT - 1) / a.CT);
  }
  a.cph_off[q] = off;
}

// Phase 3, every thread: each token into its minibatch's list.
template <class Ops>
MK_HD void plan_fill(const Plan &a, int tid, int nthr, int *fill) {
  for (int t = tid; t < a.T; t += nthr) {
    const int m = a.tok_m[t];
    a.tl[a.tl_off[m] + Ops::shared_add(&fill[m], 1)] = t;
  }
}

// ---- the persistent workgroup

// Thread 0 takes the next task of a queue, every thread gets it.
template <class Env>
MK_HD Task next_task(Env &env, int32_t *ctr, const int32_t *ph_kind, const int32_t *ph_m,
                     const int32_t *ph_off, int nph) {
  Task t{0, 0, 0, 0};
  if (env.tid() == 0) {
    const int total = ph_off[nph];
    const int i = env.atomic_add(ctr, 1);
    if (i < total) {
      int p = 0;
      while (ph_off[p + 1] <= i) p++;
      t = Task{ph_kind[p], ph_m[p], i - ph_off[p], 1};
    }
  }
  return env.bcast(t);
}

// Thread 0 alone polls *flag until it reaches `target`, with naps that grow
// to a few microseconds; the other threads wait at the barrier.  The status
// word is read every eighth poll.  Returns false (for every thread) when the
// wait failed.
template <class Env>
MK_HD bool wait_all(Env &env, const Plan &a, const int32_t *flag, int target) {
  int fail = 0;
  if (env.tid() == 0) {
    const unsigned long long t0 = env.now();
    int nap = 1;
    for (int n = 0;; n++) {
      if (env.poll(flag) >= target) break;
      if ((n & 7) == 7 &&
          (env.poll(a.status) != kStatusOk || env.now() - t0 > a.watchdog_ticks)) {
        fail = 1;
        break;
      }
      env.nap(nap);
      nap = imin(2 * nap, 4);
    }
    if (fail) env.cas(a.status, kStatusOk, kStatusTimeout);
  }
  const bool ok = env.bcast_fail(fail) == 0;
  if (ok) env.fence_acquire();
  return ok;
}

// This workgroup's writes become visible device-wide, then thread 0 adds v.
template <class Env>
MK_HD void signal_add(Env &env, int32_t *ctr, int v) {
  env.fence_release();
  env.barrier();
  if (env.tid() == 0) env.atomic_add(ctr, v);
}

// The whole life of workgroup `wg`: communication tasks first (workgroups
// below n_comm), then GEMM tiles until both queues are empty.
template <class Env, class Work>
MK_HD void run_workgroup(const Plan &a, int wg, Env &env, Work &work) {
  const int nN1 = n_cols1(a), nN2 = n_cols2(a), nN1s = n_cols1s(a);
  if (wg < a.n_comm) {
    for (;;) {
      const Task t = next_task(env, a.comm_next, a.cph_kind, a.cph_m, a.cph_off, a.n_cph);
      if (!t.ok) break;
      const int m = t.m;
      if (t.kind == CP_D) {
        if (m >= a.S) {
          const int need = (a.mt_off[m - a.S + 1] - a.mt_off[m - a.S]) * nN1;
          if (!wait_all(env, a, a.g1m_done + (m - a.S), need)) return;
        }
        const int r0 = m * a.MB + t.local * a.DCH;
        const int r1 = imin(imin(r0 + a.DCH, (m + 1) * a.MB), a.R);
        work.dispatch(m, r0, r1);
        signal_add(env, a.disp_done + m, 1);
      } else {
        for (int mm = 0; mm <= m; mm++) {
          const int need = (a.mt_off[mm + 1] - a.mt_off[mm]) * nN2;
          if (!wait_all(env, a, a.g2m_done + mm, need)) return;
        }
        if (a.Is > 0 && !wait_all(env, a, a.sg2_done, shared_row_tiles(a) * nN2)) return;
        const int b0 = a.tl_off[m] + t.local * a.CT;
        const int b1 = imin(b0 + a.CT, a.tl_off[m + 1]);
        work.combine(m, b0, b1);
        env.barrier();
      }
    }
    // the communication queue is done: help with GEMM tiles
  }
  for (;;) {
    const Task t = next_task(env, a.gemm_next, a.ph_kind, a.ph_m, a.ph_off, a.n_ph);
    if (!t.ok) break;
    if (t.kind == PH_SG1 || t.kind == PH_SG2) {
      const int nN = t.kind == PH_SG1 ? nN1s : nN2;
      const int mt = t.local / nN, nt = t.local % nN;
      if (t.kind == PH_SG2 && !wait_all(env, a, a.sg1_done + mt, nN1s)) return;
      work.tile(t.kind, 0, -1, 0, mt * kTileRows, imin(kTileRows, a.T - mt * kTileRows), mt, nt);
      signal_add(env, t.kind == PH_SG1 ? a.sg1_done + mt : a.sg2_done, 1);
    } else {
      const int nN = t.kind == PH_G1 ? nN1 : nN2;
      const int idx = a.mt_off[t.m] + t.local / nN, nt = t.local % nN;
      const int e = a.mt_list[3 * idx], row0 = a.mt_list[3 * idx + 1],
                rows = a.mt_list[3 * idx + 2];
      if (t.kind == PH_G1) {
        if (!wait_all(env, a, a.disp_done + t.m, dispatch_chunks(a, t.m))) return;
        work.tile(PH_G1, t.m, idx, e, row0, rows, -1, nt);
        env.fence_release();
        env.barrier();
        if (env.tid() == 0) {
          env.atomic_add(a.g1_done + idx, 1);
          env.atomic_add(a.g1m_done + t.m, 1);
        }
      } else {
        if (!wait_all(env, a, a.g1_done + idx, nN1)) return;
        work.tile(PH_G2, t.m, idx, e, row0, rows, -1, nt);
        signal_add(env, a.g2m_done + t.m, 1);
      }
    }
  }
}

}  // namespace mk
}  // namespace moe
