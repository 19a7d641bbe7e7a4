// Host check of the decode tile pipeline's visiting order (tile_schedule in
// gqa_paged_kv_attention_amd/csrc/tile_schedule.h, the function the kernels
// call).  Built with g++ by tests/test_tile_schedule.py, with __host__ and
// __device__ defined away.
//
// For both modes and every tile range [it0, it1) with stride `step` that the
// decode kernels can hand a wave (step 1: a wave's own consecutive tiles;
// step 2..8: tiles shared round-robin by the waves of a work-group), it checks:
//  - every tile it0, it0 + step, ... < it1 is computed exactly once, and no
//    other tile is computed;
//  - a compute of register set r computes the tile whose pages were fetched
//    into the page set that set r was last loaded from, and set r has not been
//    reloaded since (nothing overwrites registers before they are used);
//  - every fetched tile lies in [it0, last], last being the range's final
//    visited tile (page lookups never leave the range).
// Prints "ok <cases>" on success, or the first failing case.
#include <cstdio>
#include <cstdlib>

#include "tile_schedule.h"

namespace {

struct Check {
  int it0, it1, step, mode;
  int last;
  int page_tile[2] = {-1, -1};       // tile whose ids are in page set p
  int reg_tile[2] = {-1, -1};        // tile loaded into register set r
  bool reg_used[2] = {true, true};   // set r computed since its last load
  int computed[256] = {};
  bool failed = false;
  char why[160] = {};

  void fail(const char* msg, int a, int b) {
    if (!failed) std::snprintf(why, sizeof why, "%s (%d, %d)", msg, a, b);
    failed = true;
  }
};

bool run_case(int it0, int it1, int step, gqa::TileScheduleMode mode, Check& c) {
  c.it0 = it0;
  c.it1 = it1;
  c.step = step;
  c.mode = mode;
  c.last = it1 > it0 ? it0 + (it1 - 1 - it0) / step * step : it0;
  auto fetch = [&](int p, int tile) {
    if (p < 0 || p > 1) c.fail("page set out of range", p, tile);
    if (tile < it0 || tile > c.last) c.fail("fetch outside the range", tile, c.last);
    c.page_tile[p & 1] = tile;
  };
  auto load = [&](int r, int p) {
    if (r < 0 || r > 1 || p < 0 || p > 1) c.fail("set out of range", r, p);
    if (c.page_tile[p & 1] < 0) c.fail("load from an unfetched page set", r, p);
    c.reg_tile[r & 1] = c.page_tile[p & 1];
    c.reg_used[r & 1] = false;
  };
  auto compute = [&](int r, int tile) {
    if (r < 0 || r > 1) c.fail("register set out of range", r, tile);
    if (c.reg_used[r & 1]) c.fail("compute of a set not loaded since its last compute", r, tile);
    if (c.reg_tile[r & 1] != tile) c.fail("set holds another tile", c.reg_tile[r & 1], tile);
    if (tile < 0 || tile >= 256) c.fail("tile index out of range", tile, 0);
    else c.computed[tile] += 1;
    c.reg_used[r & 1] = true;
  };
  gqa::tile_schedule(it0, it1, step, mode, fetch, load, compute);
  for (int t = 0; t < 256; ++t) {
    const bool visited = t >= it0 && t < it1 && (t - it0) % step == 0;
    if (c.computed[t] != (visited ? 1 : 0)) c.fail("tile computed a wrong number of times", t, c.computed[t]);
  }
  return !c.failed;
}

}  // namespace

int main() {
  int cases = 0;
  for (int mode = 0; mode < 2; ++mode)
    for (int step = 1; step <= 8; ++step)
      for (int it0 = 0; it0 < 24; ++it0)
        for (int it1 = 0; it1 <= 120; ++it1) {
          Check c;
          ++cases;
          if (!run_case(it0, it1, step, static_cast<gqa::TileScheduleMode>(mode), c)) {
            std::printf("FAIL mode=%d step=%d it0=%d it1=%d: %s\n", mode, step, it0, it1, c.why);
            return 1;
          }
        }
  std::printf("ok %d\n", cases);
  return 0;
}
