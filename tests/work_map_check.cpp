// Host check of the decode grid's pairing map (paired_unit in
// gqa_paged_kv_attention_amd/csrc/work_map.h, the function the kernels call).
// Built with g++ by tests/test_tile_schedule.py, with __host__ and __device__
// defined away.
//
// For every even grid size N up to 4096 it checks that the ids map one to one
// onto (unit, half) pairs, unit in [0, N / 2), half in {0, 1}, and that within
// the ids [0, 16 floor(N / 16)) the two halves of each unit share id mod 8 (one
// XCD).  Prints "ok <grids>" on success, or the first failing grid.
#include <cstdio>
#include <vector>

#include "work_map.h"

int main() {
  int grids = 0;
  for (int N = 2; N <= 4096; N += 2) {
    std::vector<int> owner(N, -1);
    const int full = N / 16 * 16;
    for (int id = 0; id < N; ++id) {
      int u = -1, h = -1;
      gqa::paired_unit(id, N, &u, &h);
      if (u < 0 || u >= N / 2 || (h != 0 && h != 1)) {
        std::printf("grid %d: id %d -> (%d, %d) out of range\n", N, id, u, h);
        return 1;
      }
      const int slot = 2 * u + h;
      if (owner[slot] >= 0) {
        std::printf("grid %d: ids %d and %d both map to (%d, %d)\n", N, owner[slot], id, u, h);
        return 1;
      }
      owner[slot] = id;
    }
    for (int u = 0; u < N / 2; ++u) {
      const int a = owner[2 * u], b = owner[2 * u + 1];
      if (a < full && b < full && a % 8 != b % 8) {
        std::printf("grid %d: unit %d on ids %d and %d (different XCDs)\n", N, u, a, b);
        return 1;
      }
      if ((a < full) != (b < full)) {
        std::printf("grid %d: unit %d split across the blocks and the remainder\n", N, u);
        return 1;
      }
    }
    ++grids;
  }
  std::printf("ok %d\n", grids);
  return 0;
}
