// CPU check of the large-M tile split and the 32-bit addressing guard of libmegamoe
// (csrc/mm_policy.h, compiled here by the host C++ compiler).  Built by tests/test_tile_policy.py
// into a shared object and called through ctypes.
#include <stdint.h>

#include "mm_policy.h"

extern "C" {

int pc_large_tiles(int c) { return mm::large_tiles(c); }
int pc_large_tile_start(int c, int i) { return mm::large_tile_start(c, i); }
int pc_large_first_ng(int c) { return mm::large_first_ng(c); }
int pc_addressable(int64_t T, int64_t H, int64_t I, int64_t k) {
  return mm::large_kernels_addressable(T, H, I, k) ? 1 : 0;
}

// Invariants of the split of an expert with c rows, for every c in [1, cmax).  Returns the first
// c that violates one (writing which into *what), or 0 when all hold.
//   1 tiles cover [0, c) in order, each non-empty and of at most 256 rows;
//   2 every tile but the last starts and ends on a 16-row group boundary;
//   3 at most one tile has an odd number of 16-row groups;
//   4 tile 0 is the largest, and large_first_ng(c) is its column groups per wave;
//   5 group counts of the tiles differ by at most 2 (pairs are dealt out evenly).
int pc_check_all(int cmax, int* what) {
  for (int c = 1; c < cmax; ++c) {
    const int n = mm::large_tiles(c);
    int prev = 0, odd = 0, gmax = 0, gmin = 1 << 30, g0 = -1;
    for (int i = 0; i < n; ++i) {
      const int m0 = mm::large_tile_start(c, i);
      const int m1 = i + 1 < n ? mm::large_tile_start(c, i + 1) : c;
      if (m0 != prev || m1 <= m0 || m1 - m0 > mm::kLargeRows) { *what = 1; return c; }
      if (m0 % 16 != 0 || (i + 1 < n && m1 % 16 != 0)) { *what = 2; return c; }
      const int g = (m1 - m0 + 15) / 16;
      odd += g & 1;
      if (i == 0) g0 = g;
      gmax = g > gmax ? g : gmax;
      gmin = g < gmin ? g : gmin;
      prev = m1;
    }
    if (prev != c) { *what = 1; return c; }
    if (odd > 1) { *what = 3; return c; }
    if (g0 != gmax || mm::large_first_ng(c) != (g0 + 1) / 2) { *what = 4; return c; }
    if (gmax - gmin > 2) { *what = 5; return c; }
  }
  *what = 0;
  return 0;
}

}  // extern "C"
