// Host model of the persistent layer forward's schedule.
//
// The plan, both task queues, their waits and their signals are the
// library's own code (mixture_experts_layer_offsets_amd/csrc/mk_schedule.h),
// compiled here for the host and run with one thread per workgroup:
//   - the environment: C++ atomics for the device-scope atomics, relaxed
//     loads for polling, fences, a 100 MHz clock from steady_clock for the
//     watchdog, and no-op barriers (a workgroup is one thread here);
//   - the work: no arithmetic; every task records that it ran and checks,
//     when it starts, that everything it reads has been produced: a G1 tile
//     needs every row of its tile dispatched, a G2 tile every G1 tile of its
//     row tile, the shared expert's down tiles its gate/up tiles, a combine
//     every G2 tile holding a row of its tokens (and the shared expert's
//     tiles of the token), a dispatch of minibatch m >= S all G1 tiles of
//     minibatch m - S (the in-flight window);
//   - residency: at most `resident` workgroups run at once, started in index
//     order as earlier ones finish (a GPU grants fewer co-resident
//     workgroups than the grid when a kernel's scratch or LDS runs out);
//   - jitter: random pauses inside tasks shake the interleavings;
//   - a lost signal (drop=1): the first completion signal of minibatch 0's
//     dispatch is dropped, so a wait can never be satisfied; every
//     workgroup must still finish, through the watchdog, with the timeout
//     status.
// After the run it checks the plan (row tiles cover the rows once, each
// inside one expert and one minibatch; every token in exactly one combine
// list, the one of its last row's minibatch) and that every task ran exactly
// once.  Prints one line: "ok ..." or "FAIL ...", exit status 0 or 1.
//
// Test infrastructure: only tests/test_mk_model.py builds and runs it.
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "../mixture_experts_layer_offsets_amd/csrc/mk_schedule.h"

using namespace moe::mk;

namespace {

struct Config {
  int T = 256, k = 2, E = 8, H = 512, I = 256, Is = 0;
  int MB = 256, S = 2, n_comm = 4, grid = 32, resident = 32;
  int DCH = 16, CT = 4;
  int drop = 0, jitter = 1;
  double zipf = 0.0;        // 0: uniform experts
  double budget_s = 30.0;   // watchdog budget per wait
  unsigned seed = 1;
};

std::mutex g_fail_mu;
std::string g_fail;
std::atomic<int> g_violations{0};

void violation(const char *fmt, int a = 0, int b = 0, int c = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, fmt, a, b, c);
  std::lock_guard<std::mutex> g(g_fail_mu);
  if (g_fail.empty()) g_fail = buf;
  g_violations++;
}

unsigned long long ticks_now() {
  using namespace std::chrono;
  return (unsigned long long)duration_cast<nanoseconds>(steady_clock::now().time_since_epoch())
             .count() /
         10;  // 100 MHz
}

struct Model;

// Drops the first increment of one counter (the lost signal).
struct Fault {
  int32_t *ptr = nullptr;
  std::atomic<bool> armed{false};
};

struct HostEnv {
  Fault *fault;
  int tid() const { return 0; }
  void barrier() const {}
  int atomic_add(int32_t *p, int v) const {
    if (p == fault->ptr && fault->armed.exchange(false)) return __atomic_load_n(p, __ATOMIC_SEQ_CST);
    return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST);
  }
  void cas(int32_t *p, int expected, int desired) const {
    __atomic_compare_exchange_n(p, &expected, desired, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST);
  }
  int poll(const int32_t *p) const { return __atomic_load_n(p, __ATOMIC_RELAXED); }
  void fence_release() const { __atomic_thread_fence(__ATOMIC_RELEASE); }
  void fence_acquire() const { __atomic_thread_fence(__ATOMIC_ACQUIRE); }
  void nap(int n) const {
    for (int i = 0; i < n; i++) std::this_thread::yield();
  }
  unsigned long long now() const { return ticks_now(); }
  Task bcast(Task t) const { return t; }
  int bcast_fail(int f) const { return f; }
};

struct HostPlanOps {
  static int shared_add(int *p, int v) {
    const int old = *p;
    *p += v;
    return old;
  }
};

struct Model {
  Config c;
  Plan pl{};
  int R = 0, max_nm = 0, max_tiles = 0;
  std::vector<int32_t> inv, offsets, mt_list, mt_off, ph, cph, tl, tl_off, tok_m, counters;
  int32_t status = kStatusOk;
  // records
  std::vector<std::atomic<int>> row_disp, g1, g2, sg1, sg2, tok_done;
  std::vector<int> row_tile;  // routed row -> row-tile index
  Fault fault;

  int nN1() const { return n_cols1(pl); }
  int nN2() const { return n_cols2(pl); }
  int nN1s() const { return n_cols1s(pl); }

  void routing(std::mt19937_64 &rng) {
    // expert per (t, j): uniform or Zipf, duplicates allowed (each (t, j) is
    // its own row); layout = stable counting sort by expert
    std::vector<double> cdf(c.E);
    double s = 0;
    for (int e = 0; e < c.E; e++) cdf[e] = (s += c.zipf > 0 ? std::pow(e + 1.0, -c.zipf) : 1.0);
    std::uniform_real_distribution<double> u(0.0, s);
    std::vector<int> idx(R);
    for (int f = 0; f < R; f++) {
      const double v = u(rng);
      int e = 0;
      while (e + 1 < c.E && cdf[e] <= v) e++;
      idx[f] = e;
    }
    std::vector<int> cnt(c.E, 0);
    for (int f = 0; f < R; f++) cnt[idx[f]]++;
    offsets.assign(c.E + 1, 0);
    for (int e = 0; e < c.E; e++) offsets[e + 1] = offsets[e] + cnt[e];
    std::vector<int> fill(offsets.begin(), offsets.end() - 1);
    inv.assign(R, 0);
    for (int f = 0; f < R; f++) inv[f] = fill[idx[f]]++;
  }

  void setup() {
    R = c.T * c.k;
    std::mt19937_64 rng(c.seed);
    routing(rng);
    pl.T = c.T; pl.H = c.H; pl.k = c.k; pl.E = c.E; pl.I = c.I; pl.Is = c.Is; pl.R = R;
    long mb = c.MB > 0 ? c.MB : 2048;
    if (mb < min_minibatch(R)) mb = min_minibatch(R);
    pl.MB = (int)(mb < R ? mb : R);
    pl.NM = (R + pl.MB - 1) / pl.MB;
    pl.S = c.S;
    pl.n_comm = c.n_comm;
    pl.DCH = c.DCH;
    pl.CT = c.CT;
    pl.watchdog_ticks = (unsigned long long)(c.budget_s * 1e8);
    pl.inv = inv.data();
    pl.offsets = offsets.data();
    max_nm = max_minibatches(R);
    max_tiles = max_row_tiles(R, c.E, max_nm);
    mt_list.assign(mt_list_words(max_tiles), -1);
    mt_off.assign(max_nm + 1, -1);
    ph.assign(ph_words(max_nm), -1);
    cph.assign(cph_words(max_nm), -1);
    tl.assign(c.T, -1);
    tl_off.assign(max_nm + 1, -1);
    tok_m.assign(c.T, -1);
    counters.assign(counter_words(c.T, max_nm, max_tiles), 12345);  // the plan zeroes them
    bind(pl, max_nm, max_tiles, mt_list.data(), mt_off.data(), ph.data(), cph.data(), tl.data(),
         tl_off.data(), tok_m.data(), counters.data(), &status);
    // the plan, as its one workgroup of 256 threads runs it (phases in order)
    std::vector<int> cnt(kMaxMinibatches), fill(kMaxMinibatches);
    for (int t = 0; t < 256; t++) plan_zero(pl, t, 256, cnt.data(), fill.data());
    for (int t = 0; t < 256; t++) plan_count<HostPlanOps>(pl, t, 256, cnt.data());
    plan_tables(pl, cnt.data());
    for (int t = 0; t < 256; t++) plan_fill<HostPlanOps>(pl, t, 256, fill.data());
    if (c.drop) {
      fault.ptr = pl.disp_done;
      fault.armed = true;
    }
  }

  // The plan's own invariants.
  bool check_plan() {
    for (int i = 0; i < pl.n_counters; i++)
      if (counters[i] != 0) return violation("counter %d not zeroed", i), false;
    const int ntiles = mt_off[pl.NM];
    if (ntiles > max_tiles) return violation("%d row tiles exceed the bound %d", ntiles, max_tiles), false;
    row_tile.assign(R, -1);
    for (int m = 0; m < pl.NM; m++) {
      for (int i = mt_off[m]; i < mt_off[m + 1]; i++) {
        const int e = mt_list[3 * i], r0 = mt_list[3 * i + 1], n = mt_list[3 * i + 2];
        if (n < 1 || n > kTileRows) return violation("tile %d has %d rows", i, n), false;
        if (r0 < m * pl.MB || r0 + n > std::min((m + 1) * pl.MB, R))
          return violation("tile %d leaves minibatch %d", i, m), false;
        if (r0 < offsets[e] || r0 + n > offsets[e + 1])
          return violation("tile %d leaves expert %d", i, e), false;
        for (int r = r0; r < r0 + n; r++) {
          if (row_tile[r] != -1) return violation("row %d in two tiles", r), false;
          row_tile[r] = i;
        }
      }
    }
    for (int r = 0; r < R; r++)
      if (row_tile[r] < 0) return violation("row %d in no tile", r), false;
    std::vector<int> seen(c.T, 0);
    for (int m = 0; m < pl.NM; m++)
      for (int b = tl_off[m]; b < tl_off[m + 1]; b++) {
        const int t = tl[b];
        if (t < 0 || t >= c.T || seen[t]++) return violation("token list entry %d bad", b), false;
        int last = 0;
        for (int j = 0; j < c.k; j++) last = std::max(last, inv[t * c.k + j]);
        if (last / pl.MB != m) return violation("token %d listed under minibatch %d", t, m), false;
      }
    if (tl_off[pl.NM] != c.T) return violation("token lists hold %d of %d", tl_off[pl.NM], c.T), false;
    return true;
  }

  void alloc_records() {
    row_disp = std::vector<std::atomic<int>>(R);
    const int ntiles = mt_off[pl.NM];
    g1 = std::vector<std::atomic<int>>((size_t)ntiles * nN1());
    g2 = std::vector<std::atomic<int>>((size_t)ntiles * nN2());
    const int MTs = shared_row_tiles(pl);
    sg1 = std::vector<std::atomic<int>>((size_t)MTs * std::max(nN1s(), 1));
    sg2 = std::vector<std::atomic<int>>((size_t)MTs * nN2());
    tok_done = std::vector<std::atomic<int>>(c.T);
  }

  bool all_once(const std::vector<std::atomic<int>> &v, const char *what) {
    for (size_t i = 0; i < v.size(); i++)
      if (v[i].load() != 1) return violation(what, (int)i, v[i].load()), false;
    return true;
  }
};

struct HostWork {
  Model &M;
  std::mt19937 rng;

  void pause() {
    if (M.c.jitter && (rng() & 15) == 0)
      std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
  }
  bool g1_of_minibatch_done(int m) {
    for (int i = M.mt_off[m]; i < M.mt_off[m + 1]; i++)
      for (int n = 0; n < M.nN1(); n++)
        if (M.g1[(size_t)i * M.nN1() + n].load() != 1) return false;
    return true;
  }
  void dispatch(int m, int r0, int r1) {
    if (m >= M.pl.S && !g1_of_minibatch_done(m - M.pl.S))
      violation("dispatch of minibatch %d before G1 of minibatch %d", m, m - M.pl.S);
    if (r0 < m * M.pl.MB || r1 > std::min((m + 1) * M.pl.MB, M.R) || r0 >= r1)
      violation("dispatch chunk [%d, %d) outside minibatch %d", r0, r1, m);
    pause();
    for (int r = r0; r < r1; r++) M.row_disp[r]++;
  }
  void combine(int m, int b0, int b1) {
    for (int b = b0; b < b1; b++) {
      const int t = M.tl[b];
      for (int j = 0; j < M.c.k; j++) {
        const int tile = M.row_tile[M.inv[t * M.c.k + j]];
        for (int n = 0; n < M.nN2(); n++)
          if (M.g2[(size_t)tile * M.nN2() + n].load() != 1)
            violation("combine of token %d before G2 tile %d, %d", t, tile, n);
      }
      if (M.c.Is > 0)
        for (int n = 0; n < M.nN2(); n++)
          if (M.sg2[(size_t)(t / kTileRows) * M.nN2() + n].load() != 1)
            violation("combine of token %d before shared down tile %d", t, n);
      M.tok_done[t]++;
    }
    (void)m;
    pause();
  }
  void tile(int kind, int m, int idx, int e, int row0, int rows, int mt, int nt) {
    (void)e;
    if (kind == PH_G1) {
      if (idx < M.mt_off[m] || idx >= M.mt_off[m + 1]) violation("G1 tile %d not in minibatch %d", idx, m);
      for (int r = row0; r < row0 + rows; r++)
        if (M.row_disp[r].load() != 1) violation("G1 tile %d before row %d is dispatched", idx, r);
      pause();
      M.g1[(size_t)idx * M.nN1() + nt]++;
    } else if (kind == PH_G2) {
      for (int n = 0; n < M.nN1(); n++)
        if (M.g1[(size_t)idx * M.nN1() + n].load() != 1)
          violation("G2 tile %d before G1 tile %d, %d", idx, idx, n);
      pause();
      M.g2[(size_t)idx * M.nN2() + nt]++;
    } else if (kind == PH_SG1) {
      pause();
      M.sg1[(size_t)mt * M.nN1s() + nt]++;
    } else {
      for (int n = 0; n < M.nN1s(); n++)
        if (M.sg1[(size_t)mt * M.nN1s() + n].load() != 1)
          violation("shared down tile %d before shared gate/up tile %d", mt, n);
      pause();
      M.sg2[(size_t)mt * M.nN2() + nt]++;
    }
  }
};

bool parse(int argc, char **argv, Config &c) {
  for (int i = 1; i < argc; i++) {
    const char *eq = strchr(argv[i], '=');
    if (!eq) return false;
    const std::string key(argv[i], eq - argv[i]);
    const char *v = eq + 1;
    if (key == "T") c.T = atoi(v);
    else if (key == "k") c.k = atoi(v);
    else if (key == "E") c.E = atoi(v);
    else if (key == "H") c.H = atoi(v);
    else if (key == "I") c.I = atoi(v);
    else if (key == "Is") c.Is = atoi(v);
    else if (key == "MB") c.MB = atoi(v);
    else if (key == "S") c.S = atoi(v);
    else if (key == "n_comm") c.n_comm = atoi(v);
    else if (key == "grid") c.grid = atoi(v);
    else if (key == "resident") c.resident = atoi(v);
    else if (key == "drop") c.drop = atoi(v);
    else if (key == "jitter") c.jitter = atoi(v);
    else if (key == "zipf") c.zipf = atof(v);
    else if (key == "budget_s") c.budget_s = atof(v);
    else if (key == "seed") c.seed = (unsigned)atoi(v);
    else return false;
  }
  return true;
}

}  // namespace

int main(int argc, char **argv) {
  Config c;
  if (!parse(argc, argv, c)) {
    fprintf(stderr, "usage: mk_model key=value ...\n");
    return 2;
  }
  Model M;
  M.c = c;
  M.setup();
  if (!M.check_plan()) {
    printf("FAIL plan: %s\n", g_fail.c_str());
    return 1;
  }
  M.alloc_records();

  // workgroups started in index order, at most `resident` at a time
  std::mutex mu;
  std::condition_variable cv;
  int running = 0;
  std::vector<std::thread> threads;
  const auto t0 = std::chrono::steady_clock::now();
  for (int wg = 0; wg < c.grid; wg++) {
    {
      std::unique_lock<std::mutex> lk(mu);
      cv.wait(lk, [&] { return running < c.resident; });
      running++;
    }
    threads.emplace_back([&, wg] {
      HostEnv env{&M.fault};
      HostWork work{M, std::mt19937(c.seed * 7919u + (unsigned)wg)};
      run_workgroup(M.pl, wg, env, work);
      std::lock_guard<std::mutex> lk(mu);
      running--;
      cv.notify_all();
    });
  }
  for (auto &t : threads) t.join();
  const double secs =
      std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();

  const int st = __atomic_load_n(&M.status, __ATOMIC_SEQ_CST);
  bool ok = g_violations.load() == 0;
  if (c.drop) {
    if (st != kStatusTimeout) violation("lost signal but status %d", st), ok = false;
  } else {
    if (st != kStatusOk) violation("status %d", st), ok = false;
    ok = ok && M.all_once(M.row_disp, "row %d dispatched %d times") &&
         M.all_once(M.g1, "G1 tile slot %d ran %d times") &&
         M.all_once(M.g2, "G2 tile slot %d ran %d times") &&
         M.all_once(M.tok_done, "token %d combined %d times");
    if (ok && c.Is > 0)
      ok = M.all_once(M.sg1, "shared gate/up slot %d ran %d times") &&
           M.all_once(M.sg2, "shared down slot %d ran %d times");
  }
  const int ntiles = M.mt_off[M.pl.NM];
  if (ok && g_violations.load() == 0) {
    printf("ok R=%d MB=%d NM=%d S=%d n_comm=%d grid=%d resident=%d row_tiles=%d gemm_tasks=%d "
           "comm_tasks=%d status=%d seconds=%.2f\n",
           M.R, M.pl.MB, M.pl.NM, M.pl.S, M.pl.n_comm, c.grid, c.resident, ntiles,
           M.pl.ph_off[M.pl.n_ph], M.pl.cph_off[M.pl.n_cph], st, secs);
    return 0;
  }
  printf("FAIL %s (violations %d, status %d, %.2f s)\n", g_fail.c_str(), g_violations.load(), st,
         secs);
  return 1;
}
