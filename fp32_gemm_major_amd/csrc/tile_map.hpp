// Workgroup -> output-tile mapping shared by every SGEMM kernel.
//
// MI355X has 8 XCDs, each with its own L2, and the dispatcher hands
// consecutive workgroup ids to the XCDs round-robin (id % 8).  The mapping
// first renumbers ids so that each XCD owns one contiguous run of the tile
// sequence, then walks the tile grid in bands of kGroupM tile rows
// (column-major inside a band).  Tiles that run at the same time on one XCD
// then share A rows and B columns in that XCD's L2.
#pragma once

#include <hip/hip_runtime.h>

namespace sgemm {

constexpr int kXcds = 8;
constexpr int kGroupM = 4;

// Bijection from workgroup id `wg` in [0, nwg) to tile (tm, tn), with
// nwg == tiles_m * tiles_n.
__host__ __device__ inline void tile_coords(int wg, int nwg, int tiles_m,
                                            int tiles_n, int& tm, int& tn) {
  const int q = nwg / kXcds, r = nwg % kXcds;
  const int xcd = wg % kXcds, idx = wg / kXcds;
  // XCD x owns ids [start(x), start(x) + count(x)), count = q + (x < r).
  const int start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  const int lin = start + idx;
  const int per_band = kGroupM * tiles_n;
  const int band = lin / per_band;
  const int first = band * kGroupM;
  const int rows = tiles_m - first < kGroupM ? tiles_m - first : kGroupM;
  const int in = lin - band * per_band;
  tm = first + in % rows;
  tn = in / rows;
}

}  // namespace sgemm
