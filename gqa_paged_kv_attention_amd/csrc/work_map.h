// Work-group -> unit maps of the decode grid, as plain integer logic that both
// the kernels and a host test (tests/work_map_check.cpp) run.
#pragma once

#include <hip/hip_runtime.h>

namespace gqa {

// Pairing of a grid of N work-groups (N even) over N / 2 units, each run twice
// (half 0 and half 1): the two halves of a unit get ids 8 apart, so that they
// share an XCD (work-group id mod 8) and its L2.  Ids [0, 16 floor(N / 16))
// pair as (i, i + 8) inside each block of 16; the remaining r ids (r even)
// pair as (full + j, full + r / 2 + j).  Sets *unit in [0, N / 2) and *half in
// {0, 1}; every (unit, half) comes from exactly one id.
__host__ __device__ __forceinline__ void paired_unit(int id, int N, int* unit, int* half) {
  const int full = N / 16 * 16;
  if (id < full) {
    *half = (id >> 3) & 1;
    *unit = ((id >> 4) << 3) | (id & 7);
  } else {
    const int r2 = (N - full) / 2;
    *half = (id - full) / r2;
    *unit = full / 2 + (id - full) % r2;
  }
}

}  // namespace gqa
