// Host/device policy of libmegamoe that needs no HIP headers: the large-M tile split of an
// expert's pool rows and the 32-bit addressing limit of the large-M kernels.  Every function is
// constexpr, so hipcc compiles it for both sides and a plain C++ compiler can check it on the CPU.
#pragma once

#include <stdint.h>

namespace mm {

constexpr int kLargeRows = 256;       // most pool rows per large-M tile

// Large-M tiling of an expert with c rows: ceil(c / 256) tiles over its G = ceil(c / 16) row
// groups of 16.  The two waves of a SIMD share a tile's groups, so a tile with an odd count
// computes one padded group; the groups are therefore dealt out in pairs (q = (G / 2) / n pairs
// each, one more for the first r = (G / 2) % n tiles) and an odd last group goes to tile r, the
// first tile with q pairs: at most one tile is odd, none has more than 16 groups, and tile 0 is
// the largest.  Tile i starts at group 2 (i q + min(i, r)) + (G odd and i > r).
constexpr int large_tiles(int c) { return (c + kLargeRows - 1) / kLargeRows; }
constexpr int large_tile_start(int c, int i) {
  const int n = large_tiles(c), g = (c + 15) / 16, pairs = g / 2, q = pairs / n, r = pairs % n;
  return 16 * (2 * (i * q + (i < r ? i : r)) + ((g & 1) && i > r ? 1 : 0));
}

// Column groups per wave of the first (largest) tile of an expert with c > 0 rows: the tile's
// 16-row groups are shared by two waves.
constexpr int large_first_ng(int c) {
  const int n = large_tiles(c), g = (c + 15) / 16, pairs = g / 2, q = pairs / n, r = pairs % n;
  const int g0 = r > 0 ? 2 * q + 2 : 2 * q + (g & 1);
  return (g0 + 1) / 2;
}

// Whether every buffer the large-M kernels address through 32-bit buffer descriptors and 32-bit
// offsets stays below 4 GiB: the activation rows x [T, H], the intermediate [T k, I] (its scales
// are smaller), the pool-order activation scale words [H / 128, T k] (4 bytes each).  The weights
// of one expert (at most 2 * 16384 * 16384 bytes) always fit.  Problems that do not fit run in
// the small-M kernels, which use 64-bit addresses.
constexpr bool large_kernels_addressable(int64_t T, int64_t H, int64_t I, int64_t k) {
  const uint64_t lim = 1ull << 32;
  const uint64_t P = (uint64_t)T * (uint64_t)k;
  return (uint64_t)T * (uint64_t)H < lim && P * (uint64_t)I < lim && (uint64_t)(H / 128) * P * 4u < lim;
}

}  // namespace mm
