// FP32 SGEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// C = alpha*A*B + beta*C, row-major, as stated on "GEMM 优化之路" (problem
// statement).  The structure keeps the page's data-reuse ladder -- block tile
// in LDS, per-wave tile in registers, double-buffered K loop, fused alpha/beta
// update -- but each level is shaped for gfx950 rather than for an FP32 CUDA
// core:
//
// * Block tile BM x BN, K step BK.  Global loads are 16-byte (dwordx4) and
//   coalesced: consecutive lanes read consecutive 16-byte pieces of an A row
//   (K-contiguous) or a B row (N-contiguous).
// * LDS keeps A as [m][k] (row stride BK+4 floats) and B as [k][n] (row stride
//   BN+4).  The A tile is not transposed: an MFMA lane consumes A values of one
//   row m over several k, so the K-contiguous layout lets one ds_read_b128
//   feed four MFMAs.  The +4 padding moves successive rows by 4 banks so the
//   16-byte reads of 16 consecutive rows hit distinct banks.
// * Each wave owns a WM x WN sub-tile made of 32x32 MFMA blocks, accumulated
//   in 16 registers per lane per block.
// * Which k an MFMA lane half uses is free as long as A and B agree: lanes
//   0-31 take k in [0, BK/2) of the tile and lanes 32-63 take [BK/2, BK), so
//   both halves read 16-byte runs of A.
// * Two LDS stages ("double buffering", page section on next optimisation
//   directions and exercise 3): the global loads of tile t+1 are issued into
//   registers before the MFMAs of tile t and written to the other stage after
//   them, with one barrier per K step.
// * Epilogue: out = alpha*acc + beta*C, C read only when beta != 0.
// * GUARD = true zero-fills every load outside the M x K / K x N windows and
//   masks stores outside M x N, so any size, leading dimension and alignment
//   works ("GEMM 优化之路", exercise 2: out-of-range loads become zeros and
//   no thread leaves before the barriers).  GUARD = false needs tile-multiple
//   sizes and 16-byte aligned A/B rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tile_map.hpp"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WM_, int WN_, int OCC_>
struct MfmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int OCC = OCC_;  // waves per SIMD the registers are sized for
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;  // 32x32 blocks per wave
  static constexpr int KH = BK / 2;                 // k per lane half per tile
  static constexpr int AS = BK + 4;                 // LDS row stride of A
  static constexpr int BS = BN + 4;                 // LDS row stride of B
  static constexpr int A_ELEMS = BM * AS;
  static constexpr int B_ELEMS = BK * BS;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 4;
  static constexpr int A_VEC = BM * BK / 4 / THREADS;  // float4 per thread
  static constexpr int B_VEC = BK * BN / 4 / THREADS;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(BK % 8 == 0, "each lane half reads whole float4 runs");
  static_assert(A_VEC >= 1 && A_VEC * THREADS * 4 == BM * BK, "A loader");
  static_assert(B_VEC >= 1 && B_VEC * THREADS * 4 == BK * BN, "B loader");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");
};

template <class T, bool GUARD>
__global__ void __launch_bounds__(T::THREADS, T::OCC)
    mfma_sgemm_kernel(int M, int N, int K, float alpha,
                      const float* __restrict__ A, int lda,
                      const float* __restrict__ B, int ldb, float beta,
                      float* __restrict__ C, int ldc, int tiles_m,
                      int tiles_n) {
  __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int li = lane & 31, lh = lane >> 5;

  // Loader coordinates: float4 number v of this thread covers
  // A row a_row[v], columns a_col..a_col+3 of the tile; B likewise.
  constexpr int A_PER_ROW = T::BK / 4, B_PER_ROW = T::BN / 4;
  constexpr int A_ROWS_PER_PASS = T::THREADS / A_PER_ROW;
  constexpr int B_ROWS_PER_PASS = T::THREADS / B_PER_ROW;
  const int a_row0 = tid / A_PER_ROW, a_col = (tid % A_PER_ROW) * 4;
  const int b_row0 = tid / B_PER_ROW, b_col = (tid % B_PER_ROW) * 4;

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x16(0.0f);

  f32x4 ra[T::A_VEC], rb[T::B_VEC];

  // Guarded kernels still use 16-byte loads for pieces that lie wholly inside
  // the operand and start on a 16-byte boundary (every piece starts at a
  // multiple of 4 elements from the tile corner, so row alignment decides).
  const bool a_vec_ok =
      (lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(A) & 15u) == 0);
  const bool b_vec_ok =
      (ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(B) & 15u) == 0);

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v) {
      const int gm = m0 + a_row0 + v * A_ROWS_PER_PASS;
      const int gk = k0 + a_col;
      const float* p = A + (size_t)gm * lda + gk;
      if (!GUARD || (a_vec_ok && gm < M && gk + 3 < K)) {
        ra[v] = *reinterpret_cast<const f32x4*>(p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ra[v][e] = (gm < M && gk + e < K) ? p[e] : 0.0f;
      }
    }
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v) {
      const int gk = k0 + b_row0 + v * B_ROWS_PER_PASS;
      const int gn = n0 + b_col;
      const float* p = B + (size_t)gk * ldb + gn;
      if (!GUARD || (b_vec_ok && gk < K && gn + 3 < N)) {
        rb[v] = *reinterpret_cast<const f32x4*>(p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rb[v][e] = (gk < K && gn + e < N) ? p[e] : 0.0f;
      }
    }
  };

  auto store_tile = [&](int stage) {
    float* As = lds + stage * T::STAGE;
    float* Bs = As + T::A_ELEMS;
#pragma unroll
    for (int v = 0; v < T::A_VEC; ++v)
      *reinterpret_cast<f32x4*>(As + (a_row0 + v * A_ROWS_PER_PASS) * T::AS +
                                a_col) = ra[v];
#pragma unroll
    for (int v = 0; v < T::B_VEC; ++v)
      *reinterpret_cast<f32x4*>(Bs + (b_row0 + v * B_ROWS_PER_PASS) * T::BS +
                                b_col) = rb[v];
  };

  auto compute_tile = [&](int stage) {
    const float* As = lds + stage * T::STAGE;
    const float* Bs = As + T::A_ELEMS;
    const float* a_base = As + (wm * T::WM + li) * T::AS + lh * T::KH;
    const float* b_base = Bs + (lh * T::KH) * T::BS + wn * T::WN + li;
#pragma unroll
    for (int q = 0; q < T::KH / 4; ++q) {
      f32x4 a[T::FM];
      float b[T::FN][4];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
        a[i] = *reinterpret_cast<const f32x4*>(a_base + i * 32 * T::AS + q * 4);
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) b[j][u] = b_base[(q * 4 + u) * T::BS + j * 32];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int j = 0; j < T::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][u], b[j][u],
                                                            acc[i][j], 0, 0, 0);
    }
  };

  const int ktiles = (K + T::BK - 1) / T::BK;
  if (ktiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int stage = kt & 1;
    const bool more = kt + 1 < ktiles;
    if (more) load_tile((kt + 1) * T::BK);
    compute_tile(stage);
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Epilogue.  Block (i, j), register r of lane (li, lh) holds
  // C(row, col) with row = 8*(r/4) + 4*lh + r%4 and col = li inside the block.
  const int row_base = m0 + wm * T::WM + lh * 4;
  const int col_base = n0 + wn * T::WN + li;
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
        const int col = col_base + j * 32;
        if (GUARD && (row >= M || col >= N)) continue;
        float* p = C + (size_t)row * ldc + col;
        float v = alpha * acc[i][j][r];
        if (beta != 0.0f) v = fmaf(beta, *p, v);
        *p = v;
      }
}

}  // namespace sgemm
