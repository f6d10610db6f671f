// C ABI of the MI355X SGEMM library: handle, argument checks, kernel table,
// kernel selection and launch on the caller's stream.  Declarations and the
// full contract are in include/sgemm.h.
//
// The host side follows the launchers of "GEMM 优化之路" (its complete
// listing: one grid of ceil(M/BM) x ceil(N/BN) blocks per call) but adds what a
// library needs: explicit leading dimensions, status codes instead of aborts,
// the caller's stream, and a choice of tile shape per problem.
#include "sgemm.h"

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>

#include "diag.hpp"
#include "lowp_gemm.hpp"
#include "lowp_gemv.hpp"
#include "mfma_sgemm.hpp"
#include "skinny_sgemm.hpp"
#include "tile_map.hpp"
#include "tiles.hpp"
#include "valu_sgemm.hpp"

using namespace sgemm;

struct sgemm_handle_s {
  int device;
  int cus;
  int variant;       // SGEMM_VARIANT_*
  int forced_kernel; // -1 = automatic
  void* workspace;   // caller's device memory for partial sums, or null
  size_t workspace_bytes;
  int forced_lowp;   // low-precision product kernel, -1 = automatic
};

namespace {

struct RunArgs {
  int ta, tb;  // A stored K x M / B stored N x K
  int M, N, K;
  float alpha, beta;
  const float* A;
  int lda;
  const float* B;
  int ldb;
  float* C;
  int ldc;
};

// What a launch needs besides the problem: the device's CU count, the
// stream-K workspace and (diagnostic runs only) the clock-stamp buffer of
// the one-tile-per-workgroup MFMA kernels.
struct LaunchCtx {
  int cus;
  float* ws;
  size_t ws_bytes;
  long long* stamps;
};

typedef hipError_t (*launch_fn)(const RunArgs&, int tiles_m, int tiles_n,
                                const LaunchCtx&, hipStream_t);

struct KernelDesc {
  const char* name;
  int variant;
  int ta, tb;  // operand storage the kernel reads
  int bm, bn;
  int bk;      // K values per LDS stage: K must be a multiple when aligned
  int threads;
  int mode;    // SGEMM_MODE_*: which problem sizes the kernel takes
  int schedule;  // SGEMM_SCHEDULE_*: one tile per workgroup, or stream-K
  int sk_per_cu;  // stream-K workgroups per CU (the grid is cus * sk_per_cu)
  launch_fn launch;
};

GemmArgs gemm_args(const RunArgs& a) {
  GemmArgs g;
  g.M = a.M;
  g.N = a.N;
  g.K = a.K;
  g.alpha = a.alpha;
  g.beta = a.beta;
  g.A = a.A;
  g.lda = a.lda;
  g.B = a.B;
  g.ldb = a.ldb;
  g.C = a.C;
  g.ldc = a.ldc;
  return g;
}

template <class T, int MODE, bool TA, bool TB>
hipError_t launch_mfma(const RunArgs& a, int tiles_m, int tiles_n,
                       const LaunchCtx& c, hipStream_t s) {
  const int nwg = tiles_m * tiles_n;
  hipLaunchKernelGGL((mfma_sgemm_kernel<T, MODE, TA, TB>), dim3(nwg),
                     dim3(T::THREADS), 0, s, gemm_args(a), tiles_m, tiles_n,
                     band_rows(tiles_m, nwg, T::BM, T::BN), c.stamps);
  return hipGetLastError();
}

// Stream-K workgroups per CU for tile T (the grid is cus * this).
template <class T>
constexpr int sk_per_cu() {
  return T::SK_PER_CU;
}

// Stream-K: the persistent kernel over the tiles x K-steps space, then the
// fixup of the split tiles.  The host has checked the workspace size.
template <class T, int MODE, bool TA, bool TB>
hipError_t launch_mfma_sk(const RunArgs& a, int tiles_m, int tiles_n,
                          const LaunchCtx& c, hipStream_t s) {
  const int tiles = tiles_m * tiles_n;
  const int grid = c.cus * sk_per_cu<T>();
  const int band = band_rows(tiles_m, tiles, T::BM, T::BN);
  const int steps = tile_k_steps<T>(a.K);
  const int dp = sk_dp_tiles(tiles, grid, steps);
  const GemmArgs g = gemm_args(a);
  hipLaunchKernelGGL((mfma_sgemm_sk_kernel<T, MODE, TA, TB>), dim3(grid),
                     dim3(T::THREADS), 0, s, g, tiles_m, tiles_n, band, steps,
                     dp, c.ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || dp == tiles) return e;
  // one 16-byte piece of a split tile per thread, up to 16 workgroups of
  // 256 per CU (a grid-stride loop covers the rest)
  const long long pieces = (long long)(tiles - dp) * (T::BM * T::BN / 4);
  const long long want = (pieces + 255) / 256;
  const int fix_grid = (int)(want < 16LL * c.cus ? want : 16LL * c.cus);
  hipLaunchKernelGGL((mfma_sgemm_fixup_kernel<T, MODE>), dim3(fix_grid),
                     dim3(256), 0, s, g, tiles_m, tiles_n, band, steps, dp,
                     grid, static_cast<const float*>(c.ws));
  return hipGetLastError();
}

template <class T, bool G>
hipError_t launch_valu(const RunArgs& a, int tiles_m, int tiles_n,
                       const LaunchCtx&, hipStream_t s) {
  const int nwg = tiles_m * tiles_n;
  hipLaunchKernelGGL((valu_sgemm_kernel<T, G>), dim3(nwg), dim3(T::THREADS),
                     0, s, a.M, a.N, a.K, a.alpha, a.A, a.lda, a.B, a.ldb,
                     a.beta, a.C, a.ldc, tiles_m, tiles_n,
                     band_rows(tiles_m, nwg));
  return hipGetLastError();
}

// Split-K ranges of a small-M launch: as many workgroups (256 columns each)
// as fit one per CU (a second round would double the time), each K range at
// least SKINNY_KC rows, and no more ranges than the workspace holds (one
// range needs none).
int skinny_splits(const RunArgs& a, const LaunchCtx& c) {
  const long long col_blocks = (a.N + SKINNY_COLS - 1) / SKINNY_COLS;
  long long s = c.cus / col_blocks;
  const long long by_k = a.K / SKINNY_KC > 1 ? a.K / SKINNY_KC : 1;
  if (s > by_k) s = by_k;
  const size_t per_split = (size_t)a.M * skinny_ws_stride(a.N) * sizeof(float);
  const long long fit = c.ws == nullptr ? 1 : (long long)(c.ws_bytes / per_split);
  if (s > fit) s = fit;
  if (s < 1) s = 1;
  const long long kps = (a.K + s - 1) / s;
  return (int)((a.K + kps - 1) / kps);  // no empty range
}

// K splits of an MFMA split-K launch (one tile row): the split count s that
// minimizes the busiest CU's work, ceil(tiles*s / cus) workgroups of
// ceil(steps/s) K steps each, with every workgroup resident at once (at most
// `resident` per CU), K ranges of at least four steps, and the partial sums
// ([split][M][N rounded up to 4] floats) inside the workspace; on a tie the
// larger s (more loads in flight).  Measured on MI355X with the 32x64 tile
// (graph replays; three workgroups fit a CU): 16 x 4096 x 4096 (64 tiles, 64
// steps) takes 16.7-16.9 us with 4 or 8 splits against 19.0 us with 12;
// 16 x 11008 x 4096 (172 tiles) 35 us with 4 splits (688 workgroups, at most
// 3 x 16 steps per CU) against 38-39 with 2 or 3 (2 x 32 or 3 x 22 steps);
// 16 x 4096 x 16384 45.6 us with 8 splits against 49.3 with 12.  *kps
// receives the range length in k.
int mfma_splits(const RunArgs& a, int bm, int bn, int bk, int resident,
                const LaunchCtx& c, int* kps) {
  const long long tiles = ((long long)(a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  const long long steps = (a.K + bk - 1) / bk;
  const size_t per_split = (size_t)a.M * skinny_ws_stride(a.N) * sizeof(float);
  const long long fit = c.ws == nullptr ? 1 : (long long)(c.ws_bytes / per_split);
  const long long cus = c.cus > 0 ? c.cus : 1;
  long long best = 1, best_work = -1;
  for (long long s = 1; s == 1 || (s <= steps / 4 && s <= fit); ++s) {
    const long long kp = (steps + s - 1) / s;
    const long long n = (steps + kp - 1) / kp;  // splits that range length gives
    const long long per_cu = (tiles * n + cus - 1) / cus;
    if (s > 1 && per_cu > resident) break;
    const long long work = per_cu * kp;
    if (best_work < 0 || work <= best_work) {
      best = n;
      best_work = work;
    }
  }
  const long long kp = (steps + best - 1) / best;
  *kps = (int)(kp * bk);
  return (int)((a.K + *kps - 1) / *kps);
}

template <class T, int MODE, bool TA, bool TB>
hipError_t launch_mfma_splitk(const RunArgs& a, int tiles_m, int tiles_n,
                              const LaunchCtx& c, hipStream_t s) {
  int kps = a.K;
  // workgroups a CU holds: waves per CU at the tile's occupancy / waves per
  // workgroup (32x64: 3, 64x64: 2)
  const int splits = mfma_splits(a, T::BM, T::BN, T::BKS, 4 * T::OCC / T::WAVES, c, &kps);
  const GemmArgs g = gemm_args(a);
  hipLaunchKernelGGL((mfma_splitk_kernel<T, MODE, TA, TB>),
                     dim3(tiles_m * tiles_n * splits), dim3(T::THREADS), 0, s, g,
                     tiles_m, tiles_n, kps, c.ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long groups = (long long)a.M * (skinny_ws_stride(a.N) / 4);
  hipLaunchKernelGGL(skinny_reduce_kernel,
                     dim3((unsigned)((groups + SKINNY_REDUCE_THREADS - 1) / SKINNY_REDUCE_THREADS)),
                     dim3(SKINNY_REDUCE_THREADS), 0, s, g, splits, static_cast<const float*>(c.ws));
  return hipGetLastError();
}

template <int MT, bool TA>
hipError_t launch_skinny_nt(const RunArgs& a, int, int, const LaunchCtx&,
                            hipStream_t s) {
  constexpr int R = skinny_nt_rows(MT);
  const int blocks = (a.N + R - 1) / R;
  hipLaunchKernelGGL((skinny_nt_kernel<MT, TA>), dim3(blocks), dim3(SKINNY_NT_THREADS),
                     0, s, gemm_args(a));
  return hipGetLastError();
}

template <int MT, bool TA>
hipError_t launch_skinny_kn(const RunArgs& a, int, int, const LaunchCtx&,
                            hipStream_t s) {
  const int blocks = (a.N + SKINNY_KN_COLS - 1) / SKINNY_KN_COLS;
  hipLaunchKernelGGL((skinny_kn_kernel<MT, TA>), dim3(blocks), dim3(SKINNY_KN_THREADS),
                     0, s, gemm_args(a));
  return hipGetLastError();
}

template <int MT, bool TA>
hipError_t launch_skinny(const RunArgs& a, int, int, const LaunchCtx& c,
                         hipStream_t s) {
  const int col_blocks = (a.N + SKINNY_COLS - 1) / SKINNY_COLS;
  const int splits = skinny_splits(a, c);
  const int kps = (a.K + splits - 1) / splits;
  const GemmArgs g = gemm_args(a);
  hipLaunchKernelGGL((skinny_sgemm_kernel<MT, TA>), dim3(col_blocks * splits),
                     dim3(SKINNY_THREADS), 0, s, g, col_blocks, kps, c.ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const long long groups = (long long)a.M * (skinny_ws_stride(a.N) / 4);
  hipLaunchKernelGGL(skinny_reduce_kernel,
                     dim3((unsigned)((groups + SKINNY_REDUCE_THREADS - 1) / SKINNY_REDUCE_THREADS)),
                     dim3(SKINNY_REDUCE_THREADS), 0, s, g, splits, static_cast<const float*>(c.ws));
  return hipGetLastError();
}


#define MFMA_ONE(T, TAG, TA, TB, MODE)                                       \
  {"mfma_" #T "_" TAG, SGEMM_VARIANT_MFMA, TA, TB, T::BM, T::BN, T::BKS,    \
   T::THREADS, MODE, SGEMM_SCHEDULE_TILES, sk_per_cu<T>(),                   \
   launch_mfma<T, MODE, TA, TB>}
#define MFMA_SK(T, TAG, TA, TB, MODE)                                        \
  {"mfma_" #T "_" TAG, SGEMM_VARIANT_MFMA, TA, TB, T::BM, T::BN, T::BKS,    \
   T::THREADS, MODE, SGEMM_SCHEDULE_STREAM_K, sk_per_cu<T>(),                \
   launch_mfma_sk<T, MODE, TA, TB>}
#define MFMA_TILES(T, PRE, TA, TB)                                           \
  MFMA_ONE(T, PRE "aligned", TA, TB, SGEMM_MODE_ALIGNED),                    \
  MFMA_ONE(T, PRE "edge", TA, TB, SGEMM_MODE_EDGE),                          \
  MFMA_ONE(T, PRE "guarded", TA, TB, SGEMM_MODE_GUARDED)
#define MFMA_STORAGE(T, PRE, TA, TB)                                         \
  MFMA_TILES(T, PRE, TA, TB),                                                \
  MFMA_SK(T, PRE "sk_aligned", TA, TB, SGEMM_MODE_ALIGNED),                  \
  MFMA_SK(T, PRE "sk_edge", TA, TB, SGEMM_MODE_EDGE)
#define MFMA_SET(T, STORAGE)                                                 \
  STORAGE(T, "", false, false),                                              \
  STORAGE(T, "tn_", true, false),                                            \
  STORAGE(T, "nt_", false, true),                                            \
  STORAGE(T, "tt_", true, true)
// Tiles of fewer than 64 rows: only A stored M x K.
#define MFMA_SET_A_STORED(T, STORAGE)                                        \
  STORAGE(T, "", false, false),                                              \
  STORAGE(T, "nt_", false, true)

// Small-M kernels: bm = the most rows of C they take, bn = the columns of C
// per workgroup.  B stored K x N: one pass for up to 8 rows (32 columns per
// workgroup), K split over workgroups for up to 16 (256 columns).  With B stored N x K every workgroup reads all of A (from
// the caches), whose traffic grows with M over the few columns a workgroup
// takes: past 8 rows the MFMA split-K kernels are faster (16 x 4096 x 4096:
// 26.5 us on 16 rows against 17), so those kernels stop at 8.
#define SKINNY(MT, PRE, TA)                                                  \
  {"valu_S" #MT "x256_" PRE "small", SGEMM_VARIANT_VALU, TA, false, MT,     \
   SKINNY_COLS, SKINNY_KC, SKINNY_THREADS, SGEMM_MODE_EDGE,                  \
   SGEMM_SCHEDULE_SMALL_M, 0, launch_skinny<MT, TA>}
#define SKINNY_KN(MT, PRE, TA)                                               \
  {"valu_S" #MT "x32_" PRE "small", SGEMM_VARIANT_VALU, TA, false, MT,      \
   SKINNY_KN_COLS, SKINNY_KN_UNIT, SKINNY_KN_THREADS, SGEMM_MODE_EDGE,       \
   SGEMM_SCHEDULE_SMALL_M, 0, launch_skinny_kn<MT, TA>}
#define SKINNY_NT(MT, PRE, TA)                                               \
  {"valu_S" #MT "_" PRE "small", SGEMM_VARIANT_VALU, TA, true, MT,          \
   skinny_nt_rows(MT), SKINNY_NT_PIECE, SKINNY_NT_THREADS, SGEMM_MODE_EDGE,  \
   SGEMM_SCHEDULE_SMALL_M, 0, launch_skinny_nt<MT, TA>}
// Small M on the matrix cores with K split (edge mode): one tile row of the
// 32x64 tile (A stored M x K) or of the 64x64 tile (A stored K x M).
#define MFMA_SPLITK(T, PRE, TA, TB)                                          \
  {"mfma_" #T "_" PRE "splitk_edge", SGEMM_VARIANT_MFMA, TA, TB, T::BM,     \
   T::BN, T::BKS, T::THREADS, SGEMM_MODE_EDGE, SGEMM_SCHEDULE_SMALL_M, 0,    \
   launch_mfma_splitk<T, SGEMM_MODE_EDGE, TA, TB>}

// Largest shape first: ties in the modelled time keep the larger tile.  The
// 256x256 tile has no stream-K instances: with 128 accumulator registers per
// lane its stream-K kernel does not fit the register file, and it never
// measured fastest (the 128x128 and 64x64 stream-K kernels cover its cases).
const KernelDesc kKernels[] = {
    MFMA_SET(M256x256, MFMA_TILES),
    MFMA_SET(M256x128, MFMA_STORAGE),
    MFMA_SET(M128x128, MFMA_STORAGE),
    MFMA_SET(M64x64, MFMA_STORAGE),
    MFMA_SET_A_STORED(M32x64, MFMA_TILES),
    {"valu_V128x128_aligned", SGEMM_VARIANT_VALU, 0, 0, V128x128::BM,
     V128x128::BN, V128x128::BK, V128x128::THREADS, SGEMM_MODE_ALIGNED,
     SGEMM_SCHEDULE_TILES, 1, launch_valu<V128x128, false>},
    {"valu_V128x128_guarded", SGEMM_VARIANT_VALU, 0, 0, V128x128::BM,
     V128x128::BN, V128x128::BK, V128x128::THREADS, SGEMM_MODE_GUARDED,
     SGEMM_SCHEDULE_TILES, 1, launch_valu<V128x128, true>},
    SKINNY_KN(1, "", false), SKINNY_KN(2, "", false), SKINNY_KN(4, "", false),
    SKINNY_KN(8, "", false), SKINNY_KN(1, "tn_", true), SKINNY_KN(2, "tn_", true),
    SKINNY_KN(4, "tn_", true), SKINNY_KN(8, "tn_", true),
    SKINNY(4, "", false), SKINNY(8, "", false), SKINNY(16, "", false),
    SKINNY(4, "tn_", true), SKINNY(8, "tn_", true), SKINNY(16, "tn_", true),
    SKINNY_NT(1, "nt_", false), SKINNY_NT(2, "nt_", false), SKINNY_NT(4, "nt_", false),
    SKINNY_NT(8, "nt_", false), SKINNY_NT(1, "tt_", true), SKINNY_NT(2, "tt_", true),
    SKINNY_NT(4, "tt_", true), SKINNY_NT(8, "tt_", true),
    MFMA_SPLITK(M32x64, "", false, false), MFMA_SPLITK(M32x64, "nt_", false, true),
    MFMA_SPLITK(M64x64, "tn_", true, false), MFMA_SPLITK(M64x64, "tt_", true, true),
};
constexpr int kNumKernels = sizeof(kKernels) / sizeof(kKernels[0]);
constexpr int kChipCus = 256;

bool ptr_aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Direct loads address an operand tile as a wave-uniform base plus 32-bit
// per-lane byte offsets: the farthest element of one K step of a tile must
// lie within 4 GiB of the tile's origin.
bool offsets_fit(const KernelDesc& k, const RunArgs& a) {
  const long long a_far = a.ta ? (long long)(k.bk - 1) * a.lda + k.bm
                               : (long long)(k.bm - 1) * a.lda + k.bk;
  const long long b_far = a.tb ? (long long)(k.bn - 1) * a.ldb + k.bk
                               : (long long)(k.bk - 1) * a.ldb + k.bn;
  return 4 * a_far < (1LL << 32) && 4 * b_far < (1LL << 32);
}

// Can kernel k run these arguments?  MFMA kernels read A and B with 16-byte
// loads that need only 4-byte alignment; the VALU kernel's aligned instance
// wants 16-byte aligned rows.
// Workspace a stream-K launch of kernel k uses: two partial tiles per
// workgroup.
size_t sk_workspace_bytes(const KernelDesc& k, int cus) {
  return 2ull * (size_t)cus * k.sk_per_cu * k.bm * k.bn * sizeof(float);
}

bool kernel_fits(const KernelDesc& k, const RunArgs& a, const LaunchCtx& c) {
  if (k.ta != a.ta || k.tb != a.tb) return false;
  if (k.schedule == SGEMM_SCHEDULE_STREAM_K &&
      (a.K <= 0 || c.ws == nullptr || c.ws_bytes < sk_workspace_bytes(k, c.cus)))
    return false;
  if (k.schedule == SGEMM_SCHEDULE_SMALL_M) {
    if (a.K <= 0 || a.M > k.bm) return false;
    // (the one-pass kernels index columns and k in 32 bits, a piece past K)
    if (k.variant == SGEMM_VARIANT_VALU)
      return (k.bn != SKINNY_KN_COLS && !a.tb) ||
             (a.N <= INT_MAX - k.bn && a.K <= INT_MAX - k.bk);
    // MFMA split-K: the edge instance's conditions, and a workspace for at
    // least one set of partial sums
    const size_t part = (size_t)a.M * skinny_ws_stride(a.N) * sizeof(float);
    return c.ws != nullptr && c.ws_bytes >= part && (!a.ta || a.M >= 4) &&
           (a.tb || a.N >= 4) && offsets_fit(k, a);
  }
  switch (k.mode) {
    case SGEMM_MODE_GUARDED:
      return true;
    case SGEMM_MODE_EDGE:
      // a 16-byte unit along M (A^T) or N (B as stored) needs 4 elements
      // to clamp onto
      return (!a.ta || a.M >= 4) && (a.tb || a.N >= 4) && offsets_fit(k, a);
    default:
      if (a.M % k.bm != 0 || a.N % k.bn != 0 || a.K % k.bk != 0) return false;
      if (k.variant == SGEMM_VARIANT_VALU)
        return a.lda % 4 == 0 && a.ldb % 4 == 0 && ptr_aligned16(a.A) &&
               ptr_aligned16(a.B);
      return offsets_fit(k, a);
  }
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Launch-time model, in microseconds.  A CU holds up to R workgroups of a
// shape at once.  The first round, with c <= R of them resident, takes
// a[c-1]*K + b[c-1] us, fitted per shape from MI355X runs at K = 512 and 2048
// with exactly c tiles per CU (so b holds the launch, the pipeline fill and
// the epilogue, and the rates hold how well c workgroups hide each other's
// latency: at K = 2048 one 4-wave 128x128 tile per CU runs at 85% of peak,
// four at 93%).  Every further round of R tiles per CU takes as*K + bs, fitted
// from the difference between 8192x8192 (or 4096x8192) and 4096x4096 at
// K = 1024 and 4096: rounds after the first run at a steadier rate, higher
// than the first for the 256x128 and 64x64 tiles and lower for 128x128
// (e.g. 256x128 over 8192x8192x4096 at 96% of peak).  The operand storages
// and the edge instances run within a few percent of these.
struct ShapeModel {
  int bm, bn, resident;
  double a[4], b[4];  // first round with c resident
  double as, bs;      // each further round
};
const ShapeModel kModels[] = {
    {256, 256, 1, {0.215192}, {45.04}, 0.22295, 15.9},
    {256, 128, 2, {0.117583, 0.216994}, {18.26, 28.46}, 0.21732, 13.1},
    {128, 128, 4, {0.058030, 0.111957, 0.164966, 0.220629}, {9.41, 11.61, 15.98, 17.97},
     0.23415, 3.8},
    {64, 64, 2, {0.016331, 0.029669}, {3.96, 6.24}, 0.028646, 4.67},
    {32, 64, 3, {0.009037, 0.015286, 0.023123}, {2.75, 4.19, 4.81}, 0.024563, 2.22},
};

// The kernel's model: its shape's, or for the VALU kernel one resident tile
// at its measured 58% of peak.
ShapeModel model_of(const KernelDesc& k) {
  if (k.variant == SGEMM_VARIANT_MFMA)
    for (const ShapeModel& m : kModels)
      if (m.bm == k.bm && m.bn == k.bn) return m;
  const double a = 2.0 * k.bm * k.bn / (157.3e6 / 256 * 0.58);
  ShapeModel m = {k.bm, k.bn, 1, {a}, {10.0}, a, 2.0};
  return m;
}

constexpr double kSecondLaunchUs = 3.0;

// c tiles per CU run together, then `more` further tiles per CU in rounds of
// R (a partial last round costs its share of a round).
double rounds_us(const ShapeModel& m, int c, double more, int K) {
  double us = m.a[c - 1] * K + m.b[c - 1];
  if (more > 0) us += more / m.resident * (m.as * K + m.bs);
  return us;
}

// One-tile-per-workgroup launch: the busiest CU runs t = ceil(tiles / cus)
// tiles.  The rates above are those of full tiles, which are bound by the
// matrix cores; a launch also cannot beat reading its operands and C from
// HBM once, counted at the ~4 TB/s these kernels stream at when there is
// little work per byte (a few rows of A against a wide B), plus the launch.
// (C is counted once whatever beta is, so that a plan never depends on
// beta: sgemm_plan_handle takes none.)
double tile_cost(const KernelDesc& k, const RunArgs& a, int cus) {
  const ShapeModel m = model_of(k);
  const long long t = ceil_div(ceil_div(a.M, k.bm) * ceil_div(a.N, k.bn), cus);
  const int c = t < m.resident ? (int)t : m.resident;
  const double us = rounds_us(m, c, (double)(t - c), a.K);
  const double bytes = 4.0 * ((double)a.M * a.K + (double)a.K * a.N + (double)a.M * a.N);
  const double floor_us = 4.0 + bytes / 4e12 * 1e6;
  return us > floor_us ? us : floor_us;
}

// Stream-K launch: the tiles spread evenly over the CUs (w per CU), sk_per_cu
// workgroups at a time, 2% slower than the same tiles launched one per
// workgroup (a persistent workgroup runs its tiles' fills and epilogues in
// series), plus (when tiles are split) ~5 us for the fixup and the partial
// tiles written and read back at ~5 TB/s: about one per split tile and one
// per workgroup.
double sk_cost(const KernelDesc& k, const RunArgs& a, int cus) {
  const ShapeModel m = model_of(k);
  const long long tiles = ceil_div(a.M, k.bm) * ceil_div(a.N, k.bn);
  const int c = k.sk_per_cu < m.resident ? k.sk_per_cu : m.resident;
  const double w = (double)tiles / cus;
  double us = w <= c ? w / c * (m.a[c - 1] * a.K + m.b[c - 1])
                     : rounds_us(m, c, w - c, a.K);
  us *= 1.02;
  const int G = cus * k.sk_per_cu;
  const int steps = (int)ceil_div(a.K, k.bk);
  const long long split = tiles - sk_dp_tiles((int)tiles, G, steps);
  if (split > 0) us += 5.0 + 2.0 * (double)(split + G) * k.bm * k.bn * 4 / 5e12 * 1e6;
  return us;
}

// Small-M launch, B stored K x N (skinny_sgemm_kernel): B streamed once at
// ~4.5 TB/s when at least half the CUs have a workgroup (proportionally less
// with fewer), ~4 us of launch and fill, and with several K ranges ~3 us for
// the second kernel plus the partial sums written and read back at ~5 TB/s
// (measured on MI355X: 1 x 4096 x 4096 in 20 us, 4 x 4096 x 16384 at 5.8
// TB/s).
//
// B stored N x K (skinny_nt_kernel, one pass): ~3.3 us of launch and
// reduction, and B at a rate that falls as the kernel's rows grow (its
// loads of A and multiply-adds per byte of B): ~7.7 TB/s up to 2 rows, 7.4
// at 4 and 6.0 at 8, once 2048 waves stream it (two workgroups per CU; a
// wave streams only while K holds a piece for it).  Fitted on MI355X graph
// replays: 1 row 4096 x 4096 11.9 us, 11008 x 4096 27.0, 4096 x 14336 33.7,
// 65536 x 1024 38.5; 4 rows 4096 x 4096 12.5, 11008 x 4096 27.3; 8 rows
// 4096 x 4096 14.7, 11008 x 4096 33.4, 14336 x 4096 40.6.
double skinny_cost(const KernelDesc& k, const RunArgs& a, const LaunchCtx& c) {
  if (!a.tb && k.bn == SKINNY_KN_COLS) {
    // B stored K x N in one pass (skinny_kn_kernel): ~2.2 us, B at ~5.8
    // TB/s (5.3 with 4 rows of A, 4.4 with 8) once 2048 waves stream it.
    // Fitted on MI355X graph replays: 1 row 4096 x 4096 13.2-13.7 us, 11008
    // x 4096 32.1-33.5, 4096 x 14336 41.9-42.5; 4 rows 4096 x 4096 14.8,
    // 11008 x 4096 35.9; 8 rows 4096 x 4096 17.5.
    const double wgs = (double)ceil_div(a.N, k.bn);
    const double units = (double)ceil_div(a.K, SKINNY_KN_UNIT);
    const double waves = std::min(wgs, (double)c.cus) *
                         std::min(units, (double)SKINNY_KN_WAVES);
    const double fill = std::min(1.0, waves / (8.0 * c.cus));
    const double bw = k.bm <= 2 ? 5.8e12 : k.bm <= 4 ? 5.3e12 : 4.4e12;
    return 2.2 + (double)a.K * a.N * 4 / (bw * fill) * 1e6;
  }
  if (a.tb) {
    const double wgs = (double)ceil_div(a.N, k.bn);
    const double pieces = (double)ceil_div(a.K, SKINNY_NT_PIECE);
    const double waves = std::min(wgs, 2.0 * c.cus) *
                         std::min(pieces, (double)SKINNY_NT_WAVES);
    const double fill = std::min(1.0, waves / (8.0 * c.cus));
    const double bw = k.bm <= 2 ? 7.7e12 : k.bm <= 4 ? 7.4e12 : 6.0e12;
    return 3.3 + (double)a.K * a.N * 4 / (bw * fill) * 1e6;
  }
  const int splits = skinny_splits(a, c);
  const double wgs = (double)((a.N + SKINNY_COLS - 1) / SKINNY_COLS) * splits;
  const double fill = 2 * wgs < c.cus ? 2 * wgs / c.cus : 1.0;
  double us = 4.0 + (double)a.K * a.N * 4 / (4.5e12 * fill) * 1e6;
  if (splits > 1)
    us += 3.0 + 2.0 * splits * a.M * skinny_ws_stride(a.N) * 4.0 / 5e12 * 1e6;
  return us;
}

// MFMA split-K launch: ~6 us of launch, pipeline fill and second kernel,
// B (and A once per tile column, mostly from L2: half weight) streamed at
// ~7.5 TB/s once the workgroups fill the CUs, and the partial sums written
// and read back at ~5 TB/s.  Fitted on MI355X with the 32x64 tile, B stored
// N x K or K x N, M 1..32 (graph replays): 4096 x 4096 (64 MB of B)
// 16.2-17.4 us, 11008 x 4096 34.7-36.2 us, 14336 x 4096 38.6-39.0 us,
// 4096 x 16384 45.2-46.4 us.
double mfma_splitk_cost(const KernelDesc& k, const RunArgs& a, const LaunchCtx& c) {
  int kps = a.K;
  const int splits = mfma_splits(a, k.bm, k.bn, k.bk, model_of(k).resident, c, &kps);
  const double wgs = (double)((a.M + k.bm - 1) / k.bm) * ((a.N + k.bn - 1) / k.bn) * splits;
  const double fill = wgs < c.cus ? wgs / c.cus : 1.0;
  const double bytes = (double)a.K * a.N * 4 + (double)a.M * a.K * 4 *
                       ((a.N + k.bn - 1) / k.bn) * 0.5;
  return 6.0 + bytes / (7.5e12 * fill) * 1e6 +
         2.0 * splits * a.M * skinny_ws_stride(a.N) * 4.0 / 5e12 * 1e6;
}

// Aligned one-tile-per-workgroup kernels of the variant and operand storage
// (the tile shapes).
bool is_shape(const KernelDesc& k, int variant, const RunArgs& a) {
  return k.variant == variant && k.mode == SGEMM_MODE_ALIGNED &&
         k.schedule == SGEMM_SCHEDULE_TILES && k.ta == a.ta && k.tb == a.tb;
}

// Instance of tile shape `shape` (an aligned kernel id) with this schedule
// for these arguments: the first of its aligned, edge and guarded instances
// that can run them.
int instance_for(int shape, const RunArgs& a, const LaunchCtx& c,
                 int schedule = SGEMM_SCHEDULE_TILES) {
  const KernelDesc& s = kKernels[shape];
  for (int mode = SGEMM_MODE_ALIGNED; mode <= SGEMM_MODE_GUARDED; ++mode) {
    for (int i = 0; i < kNumKernels; ++i) {
      const KernelDesc& k = kKernels[i];
      if (k.mode == mode && k.schedule == schedule && k.variant == s.variant &&
          k.ta == s.ta && k.tb == s.tb && k.bm == s.bm && k.bn == s.bn &&
          k.bk == s.bk && k.threads == s.threads && kernel_fits(k, a, c))
        return i;
    }
  }
  return SGEMM_ERR_UNSUPPORTED;
}

// Columns [n0, n0 + n) of the problem as a problem of its own.
RunArgs column_part(const RunArgs& a, int n0, int n) {
  RunArgs p = a;
  p.N = n;
  p.B = a.tb ? a.B + (size_t)n0 * a.ldb : a.B + n0;
  p.C = a.C + n0;
  return p;
}

// One sgemm_run is one or two launches over column ranges of C.
struct Launch {
  int kernel, n0, n;
};
struct Plan {
  int count;
  Launch part[2];
};

// Pick the launch plan with the lowest modelled time.  A single launch uses
// the best tile shape.  When that leaves the last round of workgroups part
// empty, the columns can instead be split: the first launch covers whole
// rounds of a large tile (a multiple of `cus` tiles) and the second the
// remaining columns with any shape (each launch pays its own fixed time in
// the model).  With a workspace, a stream-K launch of any shape is a third
// kind of plan.
int make_plan(int variant, const RunArgs& a, const LaunchCtx& ctx, Plan* plan) {
  const int cus = ctx.cus;
  const bool any_variant = variant == SGEMM_VARIANT_AUTO;
  if (any_variant) variant = SGEMM_VARIANT_MFMA;
  if (variant != SGEMM_VARIANT_MFMA && variant != SGEMM_VARIANT_VALU)
    return SGEMM_ERR_VALUE;
  // the small-M kernel for these arguments: the cheapest by the models of
  // the vector-ALU ones (AUTO and VALU variants) and the MFMA split-K ones
  // (AUTO and MFMA); on a tie the earlier in the table, i.e. fewer rows
  int skinny = -1;
  double skinny_us = 0.0;
  for (int i = 0; i < kNumKernels; ++i) {
    const KernelDesc& k = kKernels[i];
    if (k.schedule != SGEMM_SCHEDULE_SMALL_M || !kernel_fits(k, a, ctx)) continue;
    const bool valu = k.variant == SGEMM_VARIANT_VALU;
    if (valu ? !(any_variant || variant == SGEMM_VARIANT_VALU) : variant != SGEMM_VARIANT_MFMA)
      continue;
    const double us = valu ? skinny_cost(k, a, ctx) : mfma_splitk_cost(k, a, ctx);
    if (skinny < 0 || us < skinny_us) {
      skinny = i;
      skinny_us = us;
    }
  }
  int best = -1;
  double best_cost = 0.0;
  for (int i = 0; i < kNumKernels; ++i) {
    if (!is_shape(kKernels[i], variant, a)) continue;
    const double c = tile_cost(kKernels[i], a, cus);
    if (best < 0 || c < best_cost) {
      best = i;
      best_cost = c;
    }
  }
  if (best < 0) {  // e.g. VALU with transposes
    if (skinny < 0) return SGEMM_ERR_UNSUPPORTED;
    plan->count = 1;
    plan->part[0] = Launch{skinny, 0, a.N};
    return SGEMM_OK;
  }
  plan->count = 1;
  plan->part[0] = Launch{instance_for(best, a, ctx), 0, a.N};
  if (plan->part[0].kernel < 0) return plan->part[0].kernel;
  if (a.K <= 0 || a.M <= 0) return SGEMM_OK;
  for (int i = 0; i < kNumKernels; ++i) {
    const KernelDesc& k1 = kKernels[i];
    if (!is_shape(k1, variant, a)) continue;
    const long long tm1 = ceil_div(a.M, k1.bm);
    const int tn1 = a.N / k1.bn;
    for (int nt = 1; nt < tn1; ++nt) {
      if ((tm1 * nt) % cus != 0) continue;
      const int n1 = nt * k1.bn;
      const RunArgs p1 = column_part(a, 0, n1);
      const RunArgs p2 = column_part(a, n1, a.N - n1);
      const double c1 = tile_cost(k1, p1, cus);
      for (int j = 0; j < kNumKernels; ++j) {
        const KernelDesc& k2 = kKernels[j];
        if (!is_shape(k2, variant, a)) continue;
        // a second launch must win by more than the model's error
        const double c = (c1 + tile_cost(k2, p2, cus)) * 1.01 + kSecondLaunchUs;
        if (c < best_cost) {
          const int i1 = instance_for(i, p1, ctx), i2 = instance_for(j, p2, ctx);
          if (i1 < 0 || i2 < 0) continue;
          best_cost = c;
          plan->count = 2;
          plan->part[0] = Launch{i1, 0, n1};
          plan->part[1] = Launch{i2, n1, a.N - n1};
        }
      }
    }
  }
  if (ctx.ws != nullptr) {
    for (int i = 0; i < kNumKernels; ++i) {
      const KernelDesc& k = kKernels[i];
      if (!is_shape(k, variant, a)) continue;
      const double c = sk_cost(k, a, cus);
      if (c < best_cost) {
        const int id = instance_for(i, a, ctx, SGEMM_SCHEDULE_STREAM_K);
        if (id < 0) continue;
        best_cost = c;
        plan->count = 1;
        plan->part[0] = Launch{id, 0, a.N};
      }
    }
  }
  if (skinny >= 0 && skinny_us < best_cost) {
    plan->count = 1;
    plan->part[0] = Launch{skinny, 0, a.N};
  }
  return SGEMM_OK;
}

// Half-open byte range of a row-major window, or empty.
struct Range {
  uintptr_t lo, hi;
};
Range window(const void* p, int rows, int cols, int ld) {
  Range r = {0, 0};
  if (p == nullptr || rows <= 0 || cols <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + ((uintptr_t)(rows - 1) * (uintptr_t)ld + (uintptr_t)cols) * 4u;
  return r;
}
bool overlap(Range x, Range y) {
  return x.lo < x.hi && y.lo < y.hi && x.lo < y.hi && y.lo < x.hi;
}

LaunchCtx handle_ctx(const sgemm_handle_s* h) {
  LaunchCtx c = {h->cus, static_cast<float*>(h->workspace), h->workspace_bytes, nullptr};
  return c;
}

// The plan sgemm_run_ex follows on handle h: the forced kernel, or the
// cheapest plan for the handle's variant, CU count and workspace.
int handle_plan(const sgemm_handle_s* h, const RunArgs& a, const LaunchCtx& ctx,
                Plan* plan) {
  if (h->forced_kernel >= 0) {
    if (!kernel_fits(kKernels[h->forced_kernel], a, ctx)) return SGEMM_ERR_UNSUPPORTED;
    plan->count = 1;
    plan->part[0] = Launch{h->forced_kernel, 0, a.N};
  } else {
    const int ps = make_plan(h->variant, a, ctx, plan);
    if (ps != SGEMM_OK) return ps;
  }
  for (int p = 0; p < plan->count; ++p) {
    const KernelDesc& k = kKernels[plan->part[p].kernel];
    if (ceil_div(a.M, k.bm) * ceil_div(plan->part[p].n, k.bn) > INT_MAX)
      return SGEMM_ERR_UNSUPPORTED;
  }
  return SGEMM_OK;
}

int plan_out(const Plan& plan, int N, int* kernels, int* n_split) {
  if (kernels) {
    kernels[0] = plan.part[0].kernel;
    kernels[1] = plan.count > 1 ? plan.part[1].kernel : -1;
  }
  if (n_split) *n_split = plan.count > 1 ? plan.part[1].n0 : N;
  return plan.count;
}

// Launch every part of a plan on `stream`.
int launch_plan(const Plan& plan, const RunArgs& a, const LaunchCtx& ctx,
                hipStream_t stream) {
  for (int p = 0; p < plan.count; ++p) {
    const Launch& l = plan.part[p];
    const KernelDesc& k = kKernels[l.kernel];
    const RunArgs part = column_part(a, l.n0, l.n);
    if (k.launch(part, (int)ceil_div(a.M, k.bm), (int)ceil_div(l.n, k.bn), ctx,
                 stream) != hipSuccess)
      return SGEMM_ERR_HIP;
  }
  return SGEMM_OK;
}

// ---- the library's own scratch buffer (sgemm_run_ex_noalloc) ----------------
//
// A fixed device array that the stream-K and small-M kernels use in place of
// a caller's workspace.  In host code `scratch` names a host-side stand-in,
// not the device address: its address on each device is looked up once,
// with that device current (sgemm_create), and only that address is handed
// to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<float*> g_scratch_addr[kMaxDevices];

}  // namespace

static __device__ __align__(256) float scratch[SGEMM_SCRATCH_BYTES / sizeof(float)];

namespace {

// Look up `scratch` on device `dev` (which must be current) unless done.
// Returns SGEMM_OK or SGEMM_ERR_HIP; a failed lookup is tried again on the
// next call.
int scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return SGEMM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev].load() != nullptr) return SGEMM_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
    return SGEMM_ERR_HIP;
  g_scratch_addr[dev].store(static_cast<float*>(p));
  return SGEMM_OK;
}

float* scratch_of(int dev) {
  return dev >= 0 && dev < kMaxDevices ? g_scratch_addr[dev].load() : nullptr;
}

// ---- products with 16-bit or 8-bit A and B -----------------------------------

struct LpRun {
  int dt;      // SGEMM_DTYPE_*
  int ta, tb;  // A stored K x M / B stored N x K
  int M, N, K;
  float alpha, beta;
  const void* A;
  int lda;
  const void* B;
  int ldb;
  float* C;
  int ldc;
};

// A launch of the split-K kernels: K split into `splits` ranges of `kps`
// values, partial sums in `ws`.
struct LpSplit {
  int splits, kps;
  float* ws;
};

typedef hipError_t (*lp_launch_fn)(const LpRun&, int tiles_m, int tiles_n,
                                   const LpSplit&, hipStream_t);

struct LpKernelDesc {
  const char* name;
  int dt;
  int ta, tb;
  int bm, bn, bk;
  int threads;
  int mode;      // SGEMM_MODE_*
  int schedule;  // SGEMM_SCHEDULE_TILES, or SGEMM_SCHEDULE_SMALL_M
  int split;     // small M: K split over workgroups (needs the workspace)
  lp_launch_fn launch;
};

LpArgs lp_args(const LpRun& a) {
  LpArgs g;
  g.M = a.M;
  g.N = a.N;
  g.K = a.K;
  g.alpha = a.alpha;
  g.beta = a.beta;
  g.A = a.A;
  g.lda = a.lda;
  g.B = a.B;
  g.ldb = a.ldb;
  g.C = a.C;
  g.ldc = a.ldc;
  return g;
}

template <class T, int DT, int MODE, bool TA, bool TB>
hipError_t launch_lp_splitk(const LpRun& a, int tiles_m, int tiles_n,
                            const LpSplit& sp, hipStream_t s) {
  hipLaunchKernelGGL((lp_splitk_kernel<T, DT, MODE, TA, TB>),
                     dim3(tiles_m * tiles_n * sp.splits), dim3(T::THREADS), 0, s,
                     lp_args(a), tiles_m, tiles_n, sp.kps, sp.ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmArgs r;  // the reduction reads M, N, alpha, beta, C, ldc
  r.M = a.M;
  r.N = a.N;
  r.K = a.K;
  r.alpha = a.alpha;
  r.beta = a.beta;
  r.A = nullptr;
  r.lda = 0;
  r.B = nullptr;
  r.ldb = 0;
  r.C = a.C;
  r.ldc = a.ldc;
  const long long groups = (long long)a.M * (skinny_ws_stride(a.N) / 4);
  hipLaunchKernelGGL(skinny_reduce_kernel,
                     dim3((unsigned)((groups + SKINNY_REDUCE_THREADS - 1) / SKINNY_REDUCE_THREADS)),
                     dim3(SKINNY_REDUCE_THREADS), 0, s, r, sp.splits, static_cast<const float*>(sp.ws));
  return hipGetLastError();
}

template <int DT, bool TA>
hipError_t launch_lp_gemv(const LpRun& a, int, int tiles_n, const LpSplit&,
                          hipStream_t s) {
  hipLaunchKernelGGL((lp_gemv_kernel<DT, TA>), dim3(tiles_n), dim3(LPV_THREADS), 0, s,
                     lp_args(a));
  return hipGetLastError();
}

template <class T, int DT, int MODE, bool TA, bool TB>
hipError_t launch_lp(const LpRun& a, int tiles_m, int tiles_n, const LpSplit&,
                     hipStream_t s) {
  LpArgs g;
  g.M = a.M;
  g.N = a.N;
  g.K = a.K;
  g.alpha = a.alpha;
  g.beta = a.beta;
  g.A = static_cast<const uint16_t*>(a.A);
  g.lda = a.lda;
  g.B = static_cast<const uint16_t*>(a.B);
  g.ldb = a.ldb;
  g.C = a.C;
  g.ldc = a.ldc;
  const int nwg = tiles_m * tiles_n;
  hipLaunchKernelGGL((lp_gemm_kernel<T, DT, MODE, TA, TB>), dim3(nwg),
                     dim3(T::THREADS), 0, s, g, tiles_m, tiles_n,
                     band_rows(tiles_m, nwg));
  return hipGetLastError();
}

#define LP_ONE(T, DT, DTAG, STAG, TA, TB, MODE, MTAG)                        \
  {"lp_" DTAG "_" #T "_" STAG MTAG, DT, TA, TB, T::BM, T::BN,                \
   LpFmt<DT>::BKE, T::THREADS, MODE, SGEMM_SCHEDULE_TILES, 0,                \
   launch_lp<T, DT, MODE, TA, TB>}
// Split-K instances for products with few rows (edge mode only).
#define LP_SK(T, DT, DTAG, STAG, TA, TB)                                      \
  {"lp_" DTAG "_" #T "_" STAG "sk_edge", DT, TA, TB, T::BM, T::BN,           \
   LpFmt<DT>::BKE, T::THREADS, SGEMM_MODE_EDGE, SGEMM_SCHEDULE_SMALL_M, 1,    \
   launch_lp_splitk<T, DT, SGEMM_MODE_EDGE, TA, TB>}
// One-pass matrix-core kernels for at most 16 rows of A against B stored
// N x K (A in either storage): 16 columns per workgroup, all of K.
#define LP_GEMV(DT, DTAG, STAG, TA)                                          \
  {"lp_" DTAG "_G16x16_" STAG "small", DT, TA, true, LPV_MT, LPV_COLS,      \
   LpvFmt<DT>::KB, LPV_THREADS, SGEMM_MODE_EDGE, SGEMM_SCHEDULE_SMALL_M, 0,  \
   launch_lp_gemv<DT, TA>}
#define LP_SK_STORAGE(T, DT, DTAG)                                           \
  LP_SK(T, DT, DTAG, "", false, false), LP_SK(T, DT, DTAG, "tn_", true, false), \
  LP_SK(T, DT, DTAG, "nt_", false, true), LP_SK(T, DT, DTAG, "tt_", true, true)
#define LP_STORAGE(T, DT, DTAG, MODE, MTAG)                                  \
  LP_ONE(T, DT, DTAG, "", false, false, MODE, MTAG),                         \
  LP_ONE(T, DT, DTAG, "tn_", true, false, MODE, MTAG),                       \
  LP_ONE(T, DT, DTAG, "nt_", false, true, MODE, MTAG),                       \
  LP_ONE(T, DT, DTAG, "tt_", true, true, MODE, MTAG)
// Every tile in aligned instances; the 128x128 and 64x64 tiles in edge
// instances (a 256x256 edge kernel spills registers); the guarded instance
// (only the 64x64 tile) takes what the others cannot: an extent under one
// 16-byte piece (8 elements of a 16-bit format, 16 of an 8-bit one) along
// which an outer-contiguous operand's pieces run, or strides whose tile span
// passes the 32-bit offsets of the direct loads.  Every format and storage.
#define LP_FORMAT(DT, DTAG)                                                  \
  LP_STORAGE(L256x256, DT, DTAG, SGEMM_MODE_ALIGNED, "aligned"),             \
  LP_STORAGE(L128x128, DT, DTAG, SGEMM_MODE_ALIGNED, "aligned"),             \
  LP_STORAGE(L64x64, DT, DTAG, SGEMM_MODE_ALIGNED, "aligned"),               \
  LP_STORAGE(L128x128, DT, DTAG, SGEMM_MODE_EDGE, "edge"),                   \
  LP_STORAGE(L64x64, DT, DTAG, SGEMM_MODE_EDGE, "edge"),                     \
  LP_STORAGE(L64x64, DT, DTAG, SGEMM_MODE_GUARDED, "guarded"),               \
  LP_SK_STORAGE(L64x64, DT, DTAG),                                           \
  LP_GEMV(DT, DTAG, "nt_", false), LP_GEMV(DT, DTAG, "tt_", true)

const LpKernelDesc kLpKernels[] = {
    LP_FORMAT(SGEMM_DTYPE_BF16, "bf16"),
    LP_FORMAT(SGEMM_DTYPE_F16, "f16"),
    LP_FORMAT(SGEMM_DTYPE_FP8_E4M3, "e4m3"),
    LP_FORMAT(SGEMM_DTYPE_FP8_E5M2, "e5m2"),
};
constexpr int kNumLpKernels = sizeof(kLpKernels) / sizeof(kLpKernels[0]);

// Direct loads (aligned kernels, both operands in any storage): the farthest
// byte of one K step of a tile must lie within 4 GiB of the tile's origin.
int lp_elem_bytes(int dt) { return dt >= SGEMM_DTYPE_FP8_E4M3 ? 1 : 2; }

bool lp_offsets_fit(const LpKernelDesc& k, const LpRun& a) {
  const long long a_far = a.ta ? (long long)(k.bk - 1) * a.lda + k.bm
                               : (long long)(k.bm - 1) * a.lda + k.bk;
  const long long b_far = a.tb ? (long long)(k.bn - 1) * a.ldb + k.bk
                               : (long long)(k.bk - 1) * a.ldb + k.bn;
  const long long esz = lp_elem_bytes(a.dt);
  return esz * a_far < (1LL << 32) && esz * b_far < (1LL << 32);
}

// Direct loads (global_load_lds_dwordx4) take any 2-byte aligned address on
// gfx950 (checked with an in-bounds probe), so no kernel needs more than the
// 2-byte alignment every call has.
bool lp_fits(const LpKernelDesc& k, const LpRun& a) {
  if (k.dt != a.dt || k.ta != a.ta || k.tb != a.tb) return false;
  if (k.schedule == SGEMM_SCHEDULE_SMALL_M && a.M > k.bm) return false;
  // the one-pass small-M kernels take any K and any alignment, one launch
  // of ceil(N / bn) workgroups (columns and k indexed in 32 bits, a few
  // blocks past N and K)
  if (k.schedule == SGEMM_SCHEDULE_SMALL_M && !k.split)
    return a.N <= INT_MAX - k.bn && a.K <= INT_MAX - 1024;
  if (ceil_div(a.M, k.bm) * ceil_div(a.N, k.bn) > INT_MAX) return false;
  switch (k.mode) {
    case SGEMM_MODE_GUARDED:
      return true;
    case SGEMM_MODE_EDGE: {
      // an outer-contiguous 16-byte piece needs as many elements to clamp onto
      const int piece = 16 / lp_elem_bytes(a.dt);
      return a.K > 0 && (!a.ta || a.M >= piece) && (a.tb || a.N >= piece) &&
             lp_offsets_fit(k, a);
    }
    default:
      return a.K > 0 && a.M % k.bm == 0 && a.N % k.bn == 0 && a.K % k.bk == 0 &&
             lp_offsets_fit(k, a);
  }
}

// The kernel for these arguments: the largest tile (256, 128, then 64
// square) that still gives every CU a tile, else the 64x64 one -- except
// that the 256x256 tile is also taken when the 128x128 tiling needs three or
// more rounds of the CUs (one partial round of the larger tile is then the
// shorter: a 128x128 round costs about 1.4 quarters of a 256x256 one).  The
// first instance that fits, in this order: the aligned instance of that
// tile; for 256x256, the aligned 128x128 one (sizes that are multiples of
// 128 but not of 256); the edge instance (of the 128x128 tile in place of
// 256x256, which has none); the guarded 64x64 kernel.
int lp_select(const LpRun& a, int cus) {
  const long long t256 = ceil_div(a.M, 256) * ceil_div(a.N, 256);
  const long long t128 = ceil_div(a.M, 128) * ceil_div(a.N, 128);
  int bm = 64;
  if (t256 >= cus || t128 > 2LL * cus)
    bm = 256;
  else if (t128 >= cus)
    bm = 128;
  const int edge_bm = bm > 128 ? 128 : bm;
  const int order[4][2] = {{SGEMM_MODE_ALIGNED, bm},
                           {SGEMM_MODE_ALIGNED, bm > 128 ? 128 : bm},
                           {SGEMM_MODE_EDGE, edge_bm},
                           {SGEMM_MODE_GUARDED, 64}};
  for (int o = 0; o < 4; ++o)
    for (int id = 0; id < kNumLpKernels; ++id) {
      const LpKernelDesc& k = kLpKernels[id];
      if (k.schedule != SGEMM_SCHEDULE_TILES) continue;
      if (k.mode != order[o][0] || k.bm != order[o][1]) continue;
      if (lp_fits(k, a)) return id;
    }
  return -1;
}

// K splits for split-K kernel k on these arguments: with one tile row
// (M <= bm) and tiles for at most half the CUs, K is split into ranges of
// whole K steps, at least four steps each, so that the workgroups reach two
// per CU (the 64x64 tile's occupancy), as far as `ws_bytes` of workspace
// holds the partial sums ([split][M][N rounded up to 4] floats).  (With more
// tiles one tile per workgroup already streams B at 5-6 TB/s on MI355X --
// 4 x 11008 x 4096 in 15.0 us against 18.3 split -- and the partial sums
// and second kernel cost more than the extra workgroups bring.)  Returns the
// split count (1: no split) and the range length in *kps.
int lp_splits(const LpKernelDesc& k, const LpRun& a, int cus, size_t ws_bytes,
              int* kps) {
  *kps = a.K;
  if (a.M > k.bm || a.K <= 0) return 1;
  const long long tiles = ceil_div(a.M, k.bm) * ceil_div(a.N, k.bn);
  if (2 * tiles > cus) return 1;
  const long long steps = ceil_div(a.K, k.bk);
  long long s = 2LL * cus / tiles;
  if (s > steps / 4) s = steps / 4;
  const size_t per_split = (size_t)a.M * skinny_ws_stride(a.N) * sizeof(float);
  const long long fit = (long long)(ws_bytes / per_split);
  if (s > fit) s = fit;
  if (s < 2) return 1;
  *kps = (int)(ceil_div(steps, s) * k.bk);
  return (int)ceil_div(a.K, *kps);
}

// The launch sgemm_run_lowp makes on a handle: the forced kernel; else the
// one-pass small-M kernel when it fits (at most 16 rows of A, B stored N x K:
// a stream of B with no second pass, workspace or LDS tiles) and 64x64 tiles
// would fill at most half the CUs -- for 16-bit formats with more than four
// rows only if split K does not run; else
// the split-K kernel when it splits K (a workspace, few rows, few tiles);
// else lp_select's.  *splits receives the split count (1 for kernels that do
// not split K).  Returns the kernel id or a negative status.
int lp_plan(const LpRun& a, int forced, int cus, float* ws, size_t ws_bytes,
            int* splits, int* kps) {
  *splits = 1;
  *kps = a.K;
  if (forced >= 0) {
    const LpKernelDesc& k = kLpKernels[forced];
    if (!lp_fits(k, a)) return SGEMM_ERR_UNSUPPORTED;
    if (k.split) {
      if (ws == nullptr) return SGEMM_ERR_UNSUPPORTED;
      *splits = lp_splits(k, a, cus, ws_bytes, kps);
      if (*splits < 2) {  // runs as one range: still needs one partial set
        const size_t need = (size_t)a.M * skinny_ws_stride(a.N) * sizeof(float);
        if (ws_bytes < need) return SGEMM_ERR_UNSUPPORTED;
        *splits = 1;
        *kps = a.K;
      }
    }
    return forced;
  }
  // (with more tiles one tile per workgroup streams B faster: 4 x 11008 x
  // 4096 E4M3 in 9.2 us against 13.6 one-pass).  With 16-bit formats and
  // more than four rows every lane also loads as many bytes of A as of B,
  // and split K wins when a workspace allows it (16 x 4096 x 4096 bfloat16:
  // 8.9 us against 10.1 one-pass).
  int one_pass = -1;
  if (2 * ceil_div(a.M, 64) * ceil_div(a.N, 64) <= cus)
    for (int id = 0; id < kNumLpKernels && one_pass < 0; ++id) {
      const LpKernelDesc& k = kLpKernels[id];
      if (k.schedule == SGEMM_SCHEDULE_SMALL_M && !k.split && lp_fits(k, a)) one_pass = id;
    }
  if (one_pass >= 0 && (lp_elem_bytes(a.dt) == 1 || a.M <= 4 || ws == nullptr))
    return one_pass;
  if (ws != nullptr) {
    for (int id = 0; id < kNumLpKernels; ++id) {
      const LpKernelDesc& k = kLpKernels[id];
      if (!k.split || !lp_fits(k, a)) continue;
      const int n = lp_splits(k, a, cus, ws_bytes, kps);
      if (n >= 2) {
        *splits = n;
        return id;
      }
    }
  }
  *kps = a.K;
  if (one_pass >= 0) return one_pass;
  const int id = lp_select(a, cus);
  return id >= 0 ? id : SGEMM_ERR_UNSUPPORTED;
}

Range window_bytes(const void* p, int rows, int cols, int ld, unsigned elem) {
  Range r = {0, 0};
  if (p == nullptr || rows <= 0 || cols <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + ((uintptr_t)(rows - 1) * (uintptr_t)ld + (uintptr_t)cols) * elem;
  return r;
}

}  // namespace

extern "C" {

int sgemm_validate_ex(int transa, int transb, int M, int N, int K,
                      const float* A, int lda, const float* B, int ldb,
                      float beta, const float* C, int ldc) {
  if ((transa != SGEMM_OP_N && transa != SGEMM_OP_T) ||
      (transb != SGEMM_OP_N && transb != SGEMM_OP_T))
    return SGEMM_ERR_VALUE;
  if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_SIZE;
  // stored shapes: A is M x K (or K x M), B is K x N (or N x K)
  const int a_rows = transa ? K : M, a_cols = transa ? M : K;
  const int b_rows = transb ? N : K, b_cols = transb ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
      ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_LD;
  if (M == 0 || N == 0) return SGEMM_OK;  // nothing is touched
  if (C == nullptr) return SGEMM_ERR_NULL;
  if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_ERR_NULL;
  const Range rc = window(C, M, N, ldc);
  if (K > 0 && (overlap(rc, window(A, a_rows, a_cols, lda)) ||
                overlap(rc, window(B, b_rows, b_cols, ldb))))
    return SGEMM_ERR_ALIAS;
  (void)beta;
  return SGEMM_OK;
}

int sgemm_validate(int M, int N, int K, const float* A, int lda,
                   const float* B, int ldb, float beta, const float* C,
                   int ldc) {
  return sgemm_validate_ex(SGEMM_OP_N, SGEMM_OP_N, M, N, K, A, lda, B, ldb,
                           beta, C, ldc);
}

const char* sgemm_status_string(int status) {
  switch (status) {
    case SGEMM_OK: return "ok";
    case SGEMM_ERR_HANDLE: return "null handle";
    case SGEMM_ERR_SIZE: return "negative size";
    case SGEMM_ERR_LD: return "leading dimension too small";
    case SGEMM_ERR_NULL: return "null operand pointer";
    case SGEMM_ERR_HIP: return "HIP runtime error";
    case SGEMM_ERR_DEVICE: return "device not usable (needs gfx950, the handle's device)";
    case SGEMM_ERR_VALUE: return "unknown variant or kernel id";
    case SGEMM_ERR_ALIAS: return "C overlaps A or B";
    case SGEMM_ERR_UNSUPPORTED: return "forced kernel cannot run these arguments";
    case SGEMM_ERR_SCRATCH:
      return "the forced kernel needs more scratch than the library's fixed buffer holds";
    default: return "unknown status";
  }
}

int sgemm_num_kernels(void) { return kNumKernels; }

const char* sgemm_kernel_name(int id) {
  return (id >= 0 && id < kNumKernels) ? kKernels[id].name : nullptr;
}

int sgemm_kernel_info(int id, int* variant, int* bm, int* bn, int* bk,
                      int* threads, int* mode, int* transa, int* transb) {
  if (id < 0 || id >= kNumKernels) return SGEMM_ERR_VALUE;
  const KernelDesc& k = kKernels[id];
  if (variant) *variant = k.variant;
  if (transa) *transa = k.ta;
  if (transb) *transb = k.tb;
  if (bm) *bm = k.bm;
  if (bn) *bn = k.bn;
  if (bk) *bk = k.bk;
  if (threads) *threads = k.threads;
  if (mode) *mode = k.mode;
  return SGEMM_OK;
}

int sgemm_plan_ex(int variant, int transa, int transb, int M, int N, int K,
                  const float* A, int lda, const float* B, int ldb,
                  const float* C, int ldc, int* kernels, int* n_split) {
  if ((transa != SGEMM_OP_N && transa != SGEMM_OP_T) ||
      (transb != SGEMM_OP_N && transb != SGEMM_OP_T))
    return SGEMM_ERR_VALUE;
  const RunArgs a = {transa, transb, M, N, K, 1.0f, 0.0f, A, lda, B, ldb,
                     const_cast<float*>(C), ldc};
  Plan plan;
  const LaunchCtx ctx = {kChipCus, nullptr, 0, nullptr};
  const int st = make_plan(variant, a, ctx, &plan);
  if (st != SGEMM_OK) return st;
  return plan_out(plan, N, kernels, n_split);
}

int sgemm_plan_handle(sgemm_handle_t h, int transa, int transb, int M, int N,
                      int K, const float* A, int lda, const float* B, int ldb,
                      const float* C, int ldc, int* kernels, int* n_split) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  const int st = sgemm_validate_ex(transa, transb, M, N, K, A, lda, B, ldb,
                                   1.0f, C, ldc);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0) return 0;
  const RunArgs a = {transa, transb, M, N, K, 1.0f, 0.0f, A, lda, B, ldb,
                     const_cast<float*>(C), ldc};
  Plan plan;
  const int ps = handle_plan(h, a, handle_ctx(h), &plan);
  if (ps != SGEMM_OK) return ps;
  return plan_out(plan, N, kernels, n_split);
}

int sgemm_kernel_schedule(int id) {
  return (id >= 0 && id < kNumKernels) ? kKernels[id].schedule : SGEMM_ERR_VALUE;
}

int sgemm_workspace_size(sgemm_handle_t h, size_t* bytes) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  if (bytes == nullptr) return SGEMM_ERR_NULL;
  size_t most = 0;
  for (int i = 0; i < kNumKernels; ++i)
    if (kKernels[i].schedule == SGEMM_SCHEDULE_STREAM_K) {
      const size_t b = sk_workspace_bytes(kKernels[i], h->cus);
      if (b > most) most = b;
    }
  *bytes = most;
  return SGEMM_OK;
}

int sgemm_set_workspace(sgemm_handle_t h, void* workspace, size_t bytes) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  if (workspace == nullptr && bytes != 0) return SGEMM_ERR_NULL;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return SGEMM_ERR_VALUE;
  h->workspace = bytes ? workspace : nullptr;
  h->workspace_bytes = bytes;
  return SGEMM_OK;
}

int sgemm_plan(int variant, int M, int N, int K, const float* A, int lda,
               const float* B, int ldb, const float* C, int ldc,
               int* kernels, int* n_split) {
  return sgemm_plan_ex(variant, SGEMM_OP_N, SGEMM_OP_N, M, N, K, A, lda, B,
                       ldb, C, ldc, kernels, n_split);
}

int sgemm_select_kernel(int variant, int M, int N, int K, const float* A,
                        int lda, const float* B, int ldb, const float* C,
                        int ldc) {
  int kernels[2] = {-1, -1};
  const int n = sgemm_plan(variant, M, N, K, A, lda, B, ldb, C, ldc, kernels,
                           nullptr);
  return n < 0 ? n : kernels[0];
}

void sgemm_tile_coords(int wg, int nwg, int tiles_m, int tiles_n, int* tm,
                       int* tn) {
  int m = 0, n = 0;
  tile_coords(wg, nwg, tiles_m, tiles_n, band_rows(tiles_m, nwg), m, n);
  *tm = m;
  *tn = n;
}

int sgemm_diag_mfma_chain(int workgroups, int iterations, float* out,
                          hipStream_t stream) {
  if (workgroups <= 0 || iterations < 0) return SGEMM_ERR_SIZE;
  if (out == nullptr) return SGEMM_ERR_NULL;
  hipLaunchKernelGGL(mfma_chain_kernel, dim3(workgroups), dim3(kChainThreads),
                     0, stream, out, iterations, 1.0f, 1.0f);
  return hipGetLastError() == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

int sgemm_diag_wall_clock_khz(int* khz) {
  if (khz == nullptr) return SGEMM_ERR_NULL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SGEMM_ERR_DEVICE;
  if (hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return SGEMM_ERR_HIP;
  return *khz > 0 ? SGEMM_OK : SGEMM_ERR_HIP;
}

int sgemm_diag_mfma_chain_lowp(int dtype, int workgroups, int iterations,
                               float* out, hipStream_t stream) {
  if (dtype < SGEMM_DTYPE_BF16 || dtype > SGEMM_DTYPE_FP8_E5M2) return SGEMM_ERR_VALUE;
  if (workgroups <= 0 || iterations < 0) return SGEMM_ERR_SIZE;
  if (out == nullptr) return SGEMM_ERR_NULL;
  static void (*const kChains[4])(float*, int) = {
      mfma_chain16_kernel<1>, mfma_chain16_kernel<2>, mfma_chain16_kernel<3>,
      mfma_chain16_kernel<4>};
  hipLaunchKernelGGL(kChains[dtype - SGEMM_DTYPE_BF16], dim3(workgroups),
                     dim3(kChainThreads), 0, stream, out, iterations);
  return hipGetLastError() == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

int sgemm_create(sgemm_handle_t* out) {
  if (out == nullptr) return SGEMM_ERR_HANDLE;
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SGEMM_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SGEMM_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return SGEMM_ERR_DEVICE;
  // Set-up of the fixed scratch buffer on this device (once per device);
  // a failure only disables sgemm_run_ex_noalloc, which then reports it.
  (void)scratch_setup(dev);
  sgemm_handle_s* h = new (std::nothrow) sgemm_handle_s;
  if (h == nullptr) return SGEMM_ERR_HIP;
  h->device = dev;
  h->cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kChipCus;
  h->variant = SGEMM_VARIANT_AUTO;
  h->forced_kernel = -1;
  h->workspace = nullptr;
  h->workspace_bytes = 0;
  h->forced_lowp = -1;
  *out = h;
  return SGEMM_OK;
}

int sgemm_destroy(sgemm_handle_t h) {
  delete h;
  return SGEMM_OK;
}

int sgemm_set_variant(sgemm_handle_t h, int variant) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  if (variant != SGEMM_VARIANT_AUTO && variant != SGEMM_VARIANT_MFMA &&
      variant != SGEMM_VARIANT_VALU)
    return SGEMM_ERR_VALUE;
  h->variant = variant;
  return SGEMM_OK;
}

int sgemm_set_kernel(sgemm_handle_t h, int kernel_id) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  if (kernel_id < -1 || kernel_id >= kNumKernels) return SGEMM_ERR_VALUE;
  h->forced_kernel = kernel_id;
  return SGEMM_OK;
}

int sgemm_run_ex(sgemm_handle_t h, int transa, int transb, int M, int N,
                 int K, float alpha, const float* A, int lda, const float* B,
                 int ldb, float beta, float* C, int ldc, hipStream_t stream) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  const int st = sgemm_validate_ex(transa, transb, M, N, K, A, lda, B, ldb,
                                   beta, C, ldc);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0) return SGEMM_OK;
  const RunArgs a = {transa, transb, M, N, K, alpha, beta, A, lda, B, ldb,
                     C, ldc};
  const LaunchCtx ctx = handle_ctx(h);
  Plan plan;
  const int ps = handle_plan(h, a, ctx, &plan);
  if (ps != SGEMM_OK) return ps;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return SGEMM_ERR_DEVICE;
  return launch_plan(plan, a, ctx, stream);
}

int sgemm_run_ex_noalloc(sgemm_handle_t h, int transa, int transb, int M, int N,
                         int K, float alpha, const float* A, int lda, const float* B,
                         int ldb, float beta, float* C, int ldc, hipStream_t stream) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  const int st = sgemm_validate_ex(transa, transb, M, N, K, A, lda, B, ldb,
                                   beta, C, ldc);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0) return SGEMM_OK;
  float* scr = scratch_of(h->device);
  if (scr == nullptr) return SGEMM_ERR_HIP;  // the set-up lookup failed
  // A forced stream-K kernel whose partial tiles do not fit the fixed
  // buffer is refused (the planner itself only plans what fits).
  if (h->forced_kernel >= 0) {
    const KernelDesc& f = kKernels[h->forced_kernel];
    if (f.schedule == SGEMM_SCHEDULE_STREAM_K &&
        sk_workspace_bytes(f, h->cus) > SGEMM_SCRATCH_BYTES)
      return SGEMM_ERR_SCRATCH;
  }
  const RunArgs a = {transa, transb, M, N, K, alpha, beta, A, lda, B, ldb,
                     C, ldc};
  const LaunchCtx ctx = {h->cus, scr, SGEMM_SCRATCH_BYTES, nullptr};
  Plan plan;
  const int ps = handle_plan(h, a, ctx, &plan);
  if (ps != SGEMM_OK) return ps;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return SGEMM_ERR_DEVICE;
  return launch_plan(plan, a, ctx, stream);
}

int sgemm_diag_run_clocked(sgemm_handle_t h, int transa, int transb, int M, int N,
                           int K, float alpha, const float* A, int lda,
                           const float* B, int ldb, float beta, float* C, int ldc,
                           long long* stamps, int stamp_slots, hipStream_t stream) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  const int st = sgemm_validate_ex(transa, transb, M, N, K, A, lda, B, ldb,
                                   beta, C, ldc);
  if (st != SGEMM_OK) return st;
  if (stamps == nullptr) return SGEMM_ERR_NULL;
  if (M == 0 || N == 0) return SGEMM_ERR_UNSUPPORTED;
  const RunArgs a = {transa, transb, M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
  LaunchCtx ctx = handle_ctx(h);
  Plan plan;
  const int ps = handle_plan(h, a, ctx, &plan);
  if (ps != SGEMM_OK) return ps;
  const KernelDesc& k = kKernels[plan.part[0].kernel];
  if (plan.count != 1 || k.variant != SGEMM_VARIANT_MFMA ||
      k.schedule != SGEMM_SCHEDULE_TILES)
    return SGEMM_ERR_UNSUPPORTED;
  const long long nwg = ceil_div(M, k.bm) * ceil_div(N, k.bn);
  if (nwg > stamp_slots) return SGEMM_ERR_SIZE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return SGEMM_ERR_DEVICE;
  ctx.stamps = stamps;
  if (k.launch(a, (int)ceil_div(M, k.bm), (int)ceil_div(N, k.bn), ctx, stream) !=
      hipSuccess)
    return SGEMM_ERR_HIP;
  return (int)nwg;
}

int sgemm_run(sgemm_handle_t h, int M, int N, int K, float alpha,
              const float* A, int lda, const float* B, int ldb, float beta,
              float* C, int ldc, hipStream_t stream) {
  return sgemm_run_ex(h, SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, B,
                      ldb, beta, C, ldc, stream);
}

// ---- products with 16-bit or 8-bit A and B -----------------------------------

int sgemm_validate_lowp(int dtype, int transa, int transb, int M, int N, int K,
                        const void* A, int lda, const void* B, int ldb,
                        float beta, const float* C, int ldc) {
  if (dtype < SGEMM_DTYPE_BF16 || dtype > SGEMM_DTYPE_FP8_E5M2) return SGEMM_ERR_VALUE;
  if ((transa != SGEMM_OP_N && transa != SGEMM_OP_T) ||
      (transb != SGEMM_OP_N && transb != SGEMM_OP_T))
    return SGEMM_ERR_VALUE;
  if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_SIZE;
  const int a_rows = transa ? K : M, a_cols = transa ? M : K;
  const int b_rows = transb ? N : K, b_cols = transb ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
      ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_LD;
  if (M == 0 || N == 0) return SGEMM_OK;
  if (C == nullptr) return SGEMM_ERR_NULL;
  if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_ERR_NULL;
  const unsigned esz = (unsigned)lp_elem_bytes(dtype);
  if (K > 0 && (((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) &
                 (esz - 1)) != 0))
    return SGEMM_ERR_VALUE;
  const Range rc = window_bytes(C, M, N, ldc, 4);
  if (K > 0 && (overlap(rc, window_bytes(A, a_rows, a_cols, lda, esz)) ||
                overlap(rc, window_bytes(B, b_rows, b_cols, ldb, esz))))
    return SGEMM_ERR_ALIAS;
  (void)beta;
  return SGEMM_OK;
}

int sgemm_lowp_num_kernels(void) { return kNumLpKernels; }

const char* sgemm_lowp_kernel_name(int id) {
  return id >= 0 && id < kNumLpKernels ? kLpKernels[id].name : nullptr;
}

int sgemm_lowp_kernel_info(int id, int* dtype, int* bm, int* bn, int* bk,
                           int* threads, int* mode, int* transa, int* transb) {
  if (id < 0 || id >= kNumLpKernels) return SGEMM_ERR_VALUE;
  const LpKernelDesc& k = kLpKernels[id];
  if (dtype) *dtype = k.dt;
  if (bm) *bm = k.bm;
  if (bn) *bn = k.bn;
  if (bk) *bk = k.bk;
  if (threads) *threads = k.threads;
  if (mode) *mode = k.mode;
  if (transa) *transa = k.ta;
  if (transb) *transb = k.tb;
  return SGEMM_OK;
}

int sgemm_lowp_select_kernel(int dtype, int transa, int transb, int M, int N,
                             int K, const void* A, int lda, const void* B,
                             int ldb, const float* C, int ldc) {
  const int st = sgemm_validate_lowp(dtype, transa, transb, M, N, K, A, lda, B,
                                     ldb, 0.0f, C, ldc);
  if (st != SGEMM_OK) return st;
  const LpRun a = {dtype, transa, transb, M, N, K, 1.0f, 0.0f, A, lda, B, ldb,
                   const_cast<float*>(C), ldc};
  int splits = 1, kps = K;
  return lp_plan(a, -1, kChipCus, nullptr, 0, &splits, &kps);
}

int sgemm_set_lowp_kernel(sgemm_handle_t h, int kernel_id) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  if (kernel_id < -1 || kernel_id >= kNumLpKernels) return SGEMM_ERR_VALUE;
  h->forced_lowp = kernel_id;
  return SGEMM_OK;
}

int sgemm_run_lowp(sgemm_handle_t h, int dtype, int transa, int transb, int M,
                   int N, int K, float alpha, const void* A, int lda,
                   const void* B, int ldb, float beta, float* C, int ldc,
                   hipStream_t stream) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  const int st = sgemm_validate_lowp(dtype, transa, transb, M, N, K, A, lda, B,
                                     ldb, beta, C, ldc);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0) return SGEMM_OK;
  const LpRun a = {dtype, transa, transb, M, N, K, alpha, beta, A, lda, B, ldb,
                   C, ldc};
  LpSplit sp = {1, K, static_cast<float*>(h->workspace)};
  const int id = lp_plan(a, h->forced_lowp, h->cus, sp.ws, h->workspace_bytes,
                         &sp.splits, &sp.kps);
  if (id < 0) return id;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return SGEMM_ERR_DEVICE;
  const LpKernelDesc& k = kLpKernels[id];
  if (k.launch(a, (int)ceil_div(M, k.bm), (int)ceil_div(N, k.bn), sp, stream) !=
      hipSuccess)
    return SGEMM_ERR_HIP;
  return SGEMM_OK;
}

int sgemm_lowp_kernel_schedule(int id) {
  return id >= 0 && id < kNumLpKernels ? kLpKernels[id].schedule : SGEMM_ERR_VALUE;
}

int sgemm_lowp_plan_handle(sgemm_handle_t h, int dtype, int transa, int transb,
                           int M, int N, int K, const void* A, int lda,
                           const void* B, int ldb, const float* C, int ldc,
                           int* kernel, int* splits) {
  if (h == nullptr) return SGEMM_ERR_HANDLE;
  const int st = sgemm_validate_lowp(dtype, transa, transb, M, N, K, A, lda, B,
                                     ldb, 0.0f, C, ldc);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0) return SGEMM_ERR_UNSUPPORTED;
  const LpRun a = {dtype, transa, transb, M, N, K, 1.0f, 0.0f, A, lda, B, ldb,
                   const_cast<float*>(C), ldc};
  int n = 1, kps = K;
  const int id = lp_plan(a, h->forced_lowp, h->cus, static_cast<float*>(h->workspace),
                         h->workspace_bytes, &n, &kps);
  if (id < 0) return id;
  if (kernel) *kernel = id;
  if (splits) *splits = n;
  return SGEMM_OK;
}

}  // extern "C"
