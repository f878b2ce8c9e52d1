// Host-side check of the index arithmetic of the split prefill (built for
// the CPU tests; no GPU code runs): the run boundaries split_start /
// split_run, the tile order split_order / split_position, and the partial
// slots split_slot, over seeded random schedules.
//   * split_start(0) = 0, runs are non-empty and increasing, and the last
//     run ends at or past the total;
//   * split_run(x) is the run whose [start, next start) holds x;
//   * split_order is a permutation of the query tiles and split_position
//     its inverse;
//   * the parts of every cut tile get distinct slots in [0, 2 runs), and no
//     two tiles write the same slot.
// split_check returns the number of failures and describes the first.
#include <cstdio>
#include <vector>

#include "fa_fwd_kernel.hpp"

namespace {

char g_msg[256];
int g_fail = 0;

void fail(const char* what, long long a, long long b, long long c) {
  if (g_fail++ == 0) snprintf(g_msg, sizeof(g_msg), "%s (%lld, %lld, %lld)", what, a, b, c);
}

// xorshift64*, seeded: the schedules checked
unsigned long long g_state = 0x9E3779B97F4A7C15ull;
unsigned long long next() {
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 2685821657736338717ull;
}
int draw(int lo, int hi) { return lo + (int)(next() % (unsigned long long)(hi - lo + 1)); }

void check_runs(int runs, int total, int bias) {
  if (fa::split_start(0, runs, total, bias) != 0) return fail("first run starts late", runs, total, bias);
  for (int g = 0; g < runs; ++g)
    if (fa::split_start(g + 1, runs, total, bias) <= fa::split_start(g, runs, total, bias))
      return fail("empty or inverted run", runs, total, g);
  if (fa::split_start(runs, runs, total, bias) < total) return fail("runs end short", runs, total, bias);
  const int step = total > 200000 ? 7 : 1;
  for (int x = 0; x < total; x += step) {
    const int g = fa::split_run(x, runs, total, bias);
    if (g < 0 || g >= runs || fa::split_start(g, runs, total, bias) > x ||
        fa::split_start(g + 1, runs, total, bias) <= x)
      return fail("split_run", runs, total, x);
  }
}

void check_schedule(int BH, int nqt, int runs, int bias, int tile_units) {
  // tiles of tile_units * (1 + rank % 5) key tiles, laid out in split_order
  std::vector<int> u(nqt);
  int per_slice = 0;
  for (int t = 0; t < nqt; ++t) per_slice += (u[t] = tile_units * (1 + t % 5));
  const int total = per_slice * BH;
  if (total < 4 * runs) return;
  std::vector<int> owner(2 * runs, -1);
  int lin = 0;
  for (int b = 0; b < BH; ++b)
    for (int i = 0; i < nqt; ++i) {
      const int tile = b * nqt + fa::split_order(i, nqt);
      const int len = u[fa::split_order(i, nqt)];
      const int g0 = fa::split_run(lin, runs, total, bias), g1 = fa::split_run(lin + len - 1, runs, total, bias);
      if (g1 > g0)
        for (int g = g0; g <= g1; ++g) {
          const size_t slot = fa::split_slot(g, lin, runs, total, bias);
          if (slot >= (size_t)(2 * runs) || slot / 2 != (size_t)g) return fail("slot out of its run", tile, g, (long long)slot);
          if (owner[slot] != -1) return fail("slot written twice", tile, owner[slot], (long long)slot);
          owner[slot] = tile;
        }
      lin += len;
    }
}

}  // namespace

extern "C" int split_check(char* msg, int n) {
  g_fail = 0;
  g_msg[0] = 0;
  for (int nqt = 1; nqt <= 96; ++nqt) {
    std::vector<int> seen(nqt, 0);
    for (int i = 0; i < nqt; ++i) {
      const int r = fa::split_order(i, nqt);
      if (r < 0 || r >= nqt || seen[r]++) fail("split_order is not a permutation", nqt, i, r);
      else if (fa::split_position(r, nqt) != i) fail("split_position is not its inverse", nqt, i, r);
    }
  }
  for (int trial = 0; trial < 400 && !g_fail; ++trial) {
    const int runs = draw(2, 600);
    const int total = draw(4 * runs, trial % 10 == 0 ? (1 << 22) : 64 * runs);
    const int bias = draw(0, (total / runs) / 4);
    check_runs(runs, total, bias);
  }
  for (int trial = 0; trial < 300 && !g_fail; ++trial)
    check_schedule(draw(1, 32), draw(1, 40), draw(2, 512), draw(0, 3), draw(1, 20));
  if (msg && n > 0) snprintf(msg, (size_t)n, "%s", g_msg);
  return g_fail;
}
