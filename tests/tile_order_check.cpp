// Host check of the expert GEMMs' workgroup -> tile orders (tile_order.h,
// compiled here with g++).  For every shape given: each order is a bijection
// from workgroups onto tiles; in the row GEMMs' order each XCD's 32
// workgroups of a full 256-workgroup round hold a 4 x 8 block of tiles when
// the row tiles are a multiple of 4 and the column tiles of 8; in the
// weight gradients' XCD-major order XCD x (workgroup b mod 8) holds only
// groups x, x + 8, ...  Prints one line per failure, exit status 1 if any.
#include <cstdio>
#include <set>
#include <utility>
#include <vector>

#include "../mixture_experts_layer_offsets_amd/csrc/tile_order.h"

static int failures = 0;
#define CHECK(c, ...)                   \
  do {                                  \
    if (!(c)) {                         \
      std::printf(__VA_ARGS__);         \
      std::printf("\n");                \
      ++failures;                       \
    }                                   \
  } while (0)

static void row_order(int MT, int nN) {
  const int total = MT * nN;
  std::vector<int> seen(total, 0);
  std::vector<std::pair<int, int>> tile(total);
  for (int b = 0; b < total; b++) {
    int mt, nt;
    moe::tile_of_block(b, MT, nN, mt, nt);
    CHECK(mt >= 0 && mt < MT && nt >= 0 && nt < nN, "row MT=%d nN=%d b=%d -> (%d, %d) out of range",
          MT, nN, b, mt, nt);
    if (mt < 0 || mt >= MT || nt < 0 || nt >= nN) return;
    seen[mt * nN + nt]++;
    tile[b] = {mt, nt};
  }
  for (int t = 0; t < total; t++)
    CHECK(seen[t] == 1, "row MT=%d nN=%d tile %d taken %d times", MT, nN, t, seen[t]);
  if (MT % 4 != 0 || nN % 8 != 0) return;
  for (int r = 0; r + 256 <= total; r += 256)
    for (int x = 0; x < 8; x++) {
      std::set<int> rows, cols;
      for (int j = 0; j < 32; j++) {
        rows.insert(tile[r + 8 * j + x].first);
        cols.insert(tile[r + 8 * j + x].second);
      }
      const bool block = rows.size() == 4 && cols.size() == 8 &&
                         *rows.rbegin() - *rows.begin() == 3 && *cols.rbegin() - *cols.begin() == 7;
      CHECK(block, "row MT=%d nN=%d round %d XCD %d: %zu rows x %zu columns, not a 4 x 8 block", MT,
            nN, r / 256, x, rows.size(), cols.size());
    }
}

static void wgrad_order(int G, int per, bool xcd_major) {
  std::vector<int> seen(G * per, 0);
  for (int b = 0; b < G * per; b++) {
    int gi, rem;
    moe::wgrad_tile_of_block(b, per, xcd_major, gi, rem);
    CHECK(gi >= 0 && gi < G && rem >= 0 && rem < per, "wgrad G=%d per=%d xcd=%d b=%d -> (%d, %d)",
          G, per, (int)xcd_major, b, gi, rem);
    if (gi < 0 || gi >= G || rem < 0 || rem >= per) return;
    seen[gi * per + rem]++;
    if (xcd_major) CHECK(gi % 8 == b % 8, "wgrad G=%d per=%d b=%d: group %d on XCD %d", G, per, b, gi, b % 8);
  }
  for (int t = 0; t < G * per; t++)
    CHECK(seen[t] == 1, "wgrad G=%d per=%d xcd=%d tile %d taken %d times", G, per, (int)xcd_major, t,
          seen[t]);
}

int main() {
  // row tiles x column tiles: the Kimi, mid and DeepSeek-V3 GEMMs' shapes
  // (ragged row tiles of 16,384 / 24,576 / 65,536 routed rows), small and
  // odd counts, and partial last rounds
  const int mts[] = {1, 2, 3, 4, 5, 7, 8, 12, 31, 32, 33, 64, 66, 67, 68, 96, 127, 128, 130, 288};
  const int nns[] = {1, 2, 3, 5, 7, 8, 9, 11, 15, 16, 17, 24, 28, 31, 32, 56};
  for (int MT : mts)
    for (int nN : nns) row_order(MT, nN);
  // groups x tiles per group, both orders (XCD-major needs G a multiple of 8)
  const int gs[] = {1, 2, 6, 8, 16, 24, 64, 256};
  const int pers[] = {1, 3, 8, 48, 88, 224, 448};
  for (int G : gs)
    for (int per : pers) {
      wgrad_order(G, per, false);
      if (G % 8 == 0) wgrad_order(G, per, true);
    }
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
