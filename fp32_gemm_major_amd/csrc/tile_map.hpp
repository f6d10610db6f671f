// Workgroup -> output-tile mapping shared by every SGEMM kernel.
//
// MI355X has 8 XCDs, each with its own L2, and the dispatcher hands
// consecutive workgroup ids to the XCDs round-robin (id % 8).  The mapping
// first renumbers ids so that each XCD owns one contiguous run of the tile
// sequence, then walks the tile grid in bands of `band` tile rows
// (column-major inside a band).  With `band` chosen so that one XCD's share
// is a near-square block of C, the XCD reads few A rows and B columns and
// reuses them from its own L2.
#pragma once

#include <hip/hip_runtime.h>

namespace sgemm {

constexpr int kXcds = 8;

// Tile rows per band: the largest power of two g (at most the tile rows)
// with g*bm <= (share/g)*bn, i.e. one XCD's share of tiles of bm x bn a
// block of C no taller than it is wide, in elements.  Rounding toward fewer
// rows pays: each row of A gives a K step only part of a cache line (the
// rest is used a step later, and rows with power-of-two strides compete for
// the same L2 sets), while a row of k of B gives whole lines.  Measured on
// 4096^3 with 256x128 tiles: 8 rows of tiles (2048 x 1024 per XCD) fetch
// 745 MB from beyond L2 per launch, 4 rows (1024 x 2048) 603 MB, same time.
__host__ __device__ inline int band_rows(int tiles_m, int nwg, int bm = 1, int bn = 1) {
  const long long per_xcd = (nwg + kXcds - 1) / kXcds;
  int g = 1;
  while (2 * g <= tiles_m && 4LL * g * g * bm <= per_xcd * bn) g *= 2;
  return g;
}

// Tile `lin` of the band walk: bands of `band` tile rows, column-major
// inside a band, so a contiguous run of `lin` is a compact block of C.
__host__ __device__ inline void band_walk(int lin, int tiles_m, int tiles_n,
                                          int band, int& tm, int& tn) {
  const int per_band = band * tiles_n;
  const int b = lin / per_band;
  const int first = b * band;
  const int rows = tiles_m - first < band ? tiles_m - first : band;
  const int in = lin - b * per_band;
  tm = first + in % rows;
  tn = in / rows;
}

// Bijection from workgroup id `wg` in [0, nwg) to tile (tm, tn), with
// nwg == tiles_m * tiles_n and band >= 1.
__host__ __device__ inline void tile_coords(int wg, int nwg, int tiles_m,
                                            int tiles_n, int band, int& tm,
                                            int& tn) {
  const int q = nwg / kXcds, r = nwg % kXcds;
  const int xcd = wg % kXcds, idx = wg / kXcds;
  // XCD x owns ids [start(x), start(x) + count(x)), count = q + (x < r).
  const int start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  band_walk(start + idx, tiles_m, tiles_n, band, tm, tn);
}

// Workgroup position in a persistent grid of G (the stream-K kernels):
// renumbered so that the workgroups of one XCD (ids x, x+8, ...) hold one
// contiguous run of positions, and so one contiguous share of the work.
__host__ __device__ inline int xcd_position(int wg, int G) {
  return G % kXcds == 0 ? (wg % kXcds) * (G / kXcds) + wg / kXcds : wg;
}

}  // namespace sgemm
