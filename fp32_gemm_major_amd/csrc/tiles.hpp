// The tile shapes the library instantiates (their kernels are what the
// benchmark's traffic records describe, so they live apart from the host
// planner).
#pragma once

#include "mfma_sgemm.hpp"
#include "valu_sgemm.hpp"

namespace sgemm {

// MfmaTile<BM, BN, WM, WN, OCC, S, BK, KG, PF>: block tile, wave tile, the
// waves per SIMD the register budget is sized for, LDS stages, K step, K
// groups and fragment prefetch.
// 8 waves, 1 WG/CU; a K step of 32 halves the barriers per K (0.8% faster
// at 4096^3 than 16, with 128 KB of LDS for the two stages)
typedef MfmaTile<256, 256, 128, 64, 2, 2, 32> M256x256;
typedef MfmaTile<256, 128, 64, 64, 4> M256x128;   // 8 waves, 2 WG/CU
typedef MfmaTile<128, 128, 64, 64, 4> M128x128;   // 4 waves, 4 WG/CU
// Small tiles serve problems with about one tile per CU.  Four K groups of
// four waves each take a quarter of every 64-wide K step, so a CU runs 16
// waves on one tile (1024^3: 61% of peak, against 51% for one group with a
// K step of 16).  A step is only eight MFMAs per wave, so the fragments of
// the next step are read during the current one (1024^3 and 2048^3 3.4%
// faster); registers are capped for 8 waves per SIMD so that two
// workgroups still share a CU.
typedef MfmaTile<64, 64, 32, 32, 8, 2, 16, 4, 1> M64x64;  // 16 waves
// Half of that tile along M, for problems whose 64x64 tile count leaves a
// partial round of the CUs (e.g. 384 tiles on 256 CUs: half the CUs run two
// tiles while the rest idle): two waves of 32x32 per K group, four K
// groups, registers and LDS (48 KB) sized for three workgroups per CU.
// Only for A stored M x K (its rows are K-contiguous in LDS).
typedef MfmaTile<32, 64, 32, 32, 6, 2, 16, 4, 1> M32x64;  // 8 waves
typedef ValuTile<128, 128, 8> V128x128;            // 256 lanes of 8x8

}  // namespace sgemm
