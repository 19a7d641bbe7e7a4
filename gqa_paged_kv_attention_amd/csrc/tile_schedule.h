// Visiting order of a wave's key tiles (the decode tile pipeline), as plain
// integer logic that both the kernels and a host test run.
//
// A wave walks tiles it0, it0 + step, ... < it1 of one (sequence, kv head).
// The schedule issues three kinds of step through callbacks:
//   fetch(p, tile)   read the block-table entries of `tile` into page set p
//   load(r, p)       issue the K/V loads of the tile in page set p into
//                    register set r
//   compute(r, tile) Q.K^T, softmax and P.V of the tile held in register set r
// The kernels pass the real page lookups, loads and products; the host test
// (tests/tile_schedule_check.cpp) passes recorders and checks, for every
// (it0, it1, step) a work-group can produce, that each visited tile is computed
// exactly once, from registers that were loaded from that tile's pages, and
// that no load overwrites a register set before it is computed.
//
// Three modes:
//  - kSingle: one register set; fetch, load and compute each tile in turn.
//  - step 1 with kPaired: two tiles per round, both loaded, then both
//    computed; the next pair's page ids are fetched before the computes.  A
//    pair past the end repeats the last tile (loaded, never computed).
//  - otherwise (kPaired with step > 1): register sets alternate; the loads of
//    the next tile are issued before the current tile is computed.  Tiles past
//    the last are clamped to it (loaded again, never computed), so every
//    round issues the same loads.
#pragma once

#include <hip/hip_runtime.h>

namespace gqa {

enum TileScheduleMode { kSingle = 0, kPaired = 1 };

template <class Fetch, class Load, class Compute>
__host__ __device__ __forceinline__ void tile_schedule(int it0, int it1, int step, TileScheduleMode mode, Fetch fetch,
                                                       Load load, Compute compute) {
  if (it0 >= it1) return;
  if (mode == kSingle) {
    for (int it = it0; it < it1; it += step) {
      fetch(0, it);
      load(0, 0);
      compute(0, it);
    }
    return;
  }
  const int last = it0 + (it1 - 1 - it0) / step * step;     // last tile this wave visits
  auto clamp = [last](int t) { return t < last ? t : last; };
  if (step == 1) {
    fetch(0, it0);
    fetch(1, clamp(it0 + 1));
    for (int it = it0; it < it1; it += 2) {
      load(0, 0);
      load(1, 1);
      fetch(0, clamp(it + 2));
      fetch(1, clamp(it + 3));
      compute(0, it);
      if (it + 1 < it1) compute(1, it + 1);
    }
    return;
  }
  fetch(0, it0);
  load(0, 0);
  fetch(0, clamp(it0 + step));
  for (int it = it0;; it += 2 * step) {
    // set 1 <- tile it + step (clamped), then compute set 0 = tile it
    load(1, 0);
    fetch(0, clamp(it + 2 * step));
    compute(0, it);
    if (it + step > last) break;
    // set 0 <- tile it + 2 step (clamped), then compute set 1 = tile it + step
    load(0, 0);
    fetch(0, clamp(it + 3 * step));
    compute(1, it + step);
    if (it + 2 * step > last) break;
  }
}

}  // namespace gqa
